// Chunked-prefill attention over the paged cache, on the bf16 matrix cores.
//
// What is computed: the n query rows of a prompt chunk (the last n of the
// sequence's L cached tokens) attend causally to keys 0 .. L - n + i through
// the block table ("bounded 512-token chunks", mini-infer docs, "Core
// Capabilities at a Glance" table, row "Prompt Ingestion (v0.2.1)").
//
// How (gfx950):
//  * A workgroup owns 32 consecutive query positions of one sequence and one
//    kv head, with one wave per q head of the group (G waves), so every K/V
//    tile staged in LDS serves all G heads.  Long key ranges are cut into
//    pieces handled by separate workgroups (the same split-KV scheme as
//    decode) and merged by log-sum-exp afterwards.
//  * Key tiles of 64 rows stream into LDS by global_load_lds_dwordx4 in
//    pairs, four tile buffers: while one pair is computed the next is in
//    flight, and one barrier per pair publishes it and frees the buffers of
//    the pair before (where two tiles' DMAs would overflow the wait counter:
//    three buffers, two tiles in flight, one barrier per tile).  K rows are
//    stored with their 16-byte chunks XOR swizzled by row, V rows with their
//    32-byte column pairs swizzled, so the reads below hit distinct banks.
//  * S^T = K Q^T on v_mfma_f32_16x16x32_bf16: K fragments (keys x head_dim)
//    come from LDS, Q^T fragments sit in registers for the whole launch.
//    The result holds one query row per lane (row = lane % 16), so softmax
//    statistics are per lane, and the probabilities P^T become, after bf16
//    packing, the B operand of the second product without moving data:
//    the MFMA's reduction index walks the keys in the permuted order in which
//    the lanes already hold them.
//  * O^T = V^T P^T on the same MFMA: V^T fragments are read from the
//    row-major V tile with ds_read_b64_tr_b16 (a transposing LDS read), two
//    per fragment, in the same permuted key order.
//  * Online softmax in the exp2 domain with a lazily moved running max (one
//    ballot per tile; exact max and rescale only when a score exceeds the
//    max by 2^8).  Masks (causal diagonal, piece end) are applied only on
//    tiles that cross them; elsewhere the scale folds into one fma per
//    weight.  The row sums of P come from the matrix core too (a block of
//    ones times P^T), not from per-element adds.
//  * With the key range in pieces, each piece writes its normalised rows in
//    bf16 and their base-2 log-sum-exp in fp32; the merge kernel combines
//    them.
//  * fp8 pools (KV8): see prefill_kernel.
#include "pa_device.hpp"
#include "pa_kernels.hpp"

namespace pa {

namespace {

constexpr int kQRows = 32;   // query positions per workgroup (two 16-row MFMA blocks)
constexpr int kKeys = 64;    // keys per LDS tile
constexpr int KG = kKeys / 16;   // 16-key groups (MFMA key blocks) per tile
constexpr int KK = kKeys / 32;   // 32-key reduction steps of the P.V product per tile
constexpr int kTileLds = 128 * 1024;  // LDS for the K/V stages
constexpr float kSlackP = 8.f;

// v_max3_f32 without the input canonicalisation the compiler adds for fmaxf
// in IEEE mode (inputs here are matrix-core results, never signalling NaNs).
__device__ __forceinline__ float max3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

template <int D>
struct PrefillLayout {
  static constexpr int ROWB = D * 2;              // bytes of one key row (one kv head)
  static constexpr int NCH = D / 8;               // 16-byte chunks per row
  static constexpr int TILEB = kKeys * ROWB;      // bytes of one K (or V) tile
  static constexpr int NDMA = TILEB / 1024;       // DMA instructions per tensor per tile
  static constexpr int ROWS_PER_DMA = 1024 / ROWB;
  static constexpr int KSTEPS = D / 32;           // MFMA reduction steps over head_dim
  static constexpr int DBLK = D / 16;             // 16-column blocks of head_dim
};

// Stored 16-byte position of chunk c of K row r (and its inverse).
template <int D>
__device__ __forceinline__ int k_pos(int c, int r) {
  return c ^ (r & (D / 8 - 1));
}
// Stored 16-byte position of chunk c of V row r: 32-byte pairs swizzled.
template <int D>
__device__ __forceinline__ int v_pos(int c, int r) {
  return ((((c >> 1) ^ (r & (D / 16 - 1)))) << 1) | (c & 1);
}

// fp8 pools: stored 16-byte position of chunk c of K row r (rows of D
// bytes): the rows that share a 256-byte bank line get distinct positions,
// so the 8-byte K fragment reads of 16 rows hit distinct banks.
template <int D>
__device__ __forceinline__ int k_pos8(int c, int r) {
  return c ^ ((r >> (D == 128 ? 1 : 2)) & (D / 16 - 1));
}

// fp8 pools: stored 16-byte position of chunk c of V row r.  One transposing
// V read of a 16-lane group covers rows 4 q + e and 16 + 4 q + e (e < 4) of a
// 32-key step at one chunk.  D = 128: the eight rows get eight distinct
// positions.  D = 64 (four positions per row): rows e and 16 + e get distinct
// positions, and so do rows of equal parity, so no two of the eight rows meet
// in a bank whether a bank line is 128 or 256 bytes.
template <int D>
__device__ __forceinline__ int v_pos8(int c, int r) {
  return D == 128 ? c ^ ((r & 3) | ((r >> 2) & 4)) : c ^ (((r >> 1) & 1) | ((r >> 3) & 2));
}

// KV8: the pools hold fp8 codes, head-major [NB, Hkv, bs, D].  Tiles of
// codes stream into LDS and widen to bf16 in registers: K fragments after an
// 8-byte read, V^T fragments after one 8-bit transposing read that gathers a
// lane's eight keys (in the P^T key order) of its head_dim column.  k_scale
// is folded into the score scale, v_scale into the output.
template <int D, int G, bool KV8>
__global__ __launch_bounds__(64 * G) void prefill_kernel(PrefillArgs a) {
  using Lay = PrefillLayout<D>;
  constexpr int ROWB = Lay::ROWB, KS = Lay::KSTEPS;
  constexpr int DB = Lay::DBLK;
  // rows as stored and staged (one byte per element for fp8)
  constexpr int RB = KV8 ? D : ROWB;
  constexpr int NCH = RB / 16;                    // 16-byte chunks per stored row
  constexpr int TILEK = kKeys * RB;               // bytes of one staged K (or V) tile
  constexpr int NDMA = TILEK / 1024;              // DMA instructions per tensor per tile
  constexpr int RPD = 1024 / RB;                  // rows per DMA instruction
  static_assert(RPD <= 16, "a DMA instruction stays inside one 16-row group");
  // NST tile buffers.  The DMAs of a tile are issued by NI waves (a power of
  // two), NPW instructions each, so every issuing wave waits on a fixed count
  // per tile.
  constexpr int NI = G >= 4 ? 4 : (G >= 2 ? 2 : 1);
  constexpr int NPW = 2 * NDMA / NI;
  // as many stages (up to four) as kTileLds holds, fewer where the DMA
  // count of the tiles in flight behind the one waited for would overflow
  // the vmcnt field
  constexpr int STL = kTileLds / (2 * TILEK);
  constexpr int NSTL = STL < 4 ? STL : 4;
  constexpr int NST = (NSTL - 2) * NPW <= 63 ? NSTL : 3;
  static_assert(NST >= 2 && (NST - 2) * NPW <= 63, "stages and vmcnt range");
  // Four buffers: tiles go in pairs, one barrier per pair (the pair in
  // flight, 2 NPW DMAs per wave, fits the wait counter).  Otherwise one
  // barrier per tile with NST - 1 tiles in flight.
  constexpr bool PAIRS = NST == 4;
  __shared__ __attribute__((aligned(1024))) char smem[NST][2][TILEK];  // [stage][K, V]

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // q head within the group
  const int Hkv = a.num_kv_heads, Hq = a.num_q_heads;
  const int g = blockIdx.y % Hkv, piece = blockIdx.y / Hkv, b = blockIdx.z;
  const auto *cu = as_const(a.cu_seqlens_q);
  const int q0 = cu[b], n = cu[b + 1] - q0;
  const int L = as_const(a.context_lens)[b];
  const int i0 = blockIdx.x * kQRows;
  if (i0 >= n) return;
  const int pos0 = L - n + i0;                          // position of the tile's first row
  const int pmax = L - n + min(i0 + kQRows, n) - 1;     // position of its last row
  const int kbeg = piece * a.split_len;
  const int kend = min(kbeg + a.split_len, pmax + 1);
  if (kbeg >= kend) return;
  const int h = g * G + w;
  const int bs_shift = a.bs_shift, bs_mask = (1 << bs_shift) - 1;
  const auto *table = as_const(a.block_tables + (size_t)b * a.max_blocks_per_seq);
  // bf16 pools [NB, bs, Hkv, D]: token rows of one kv head are Hkv rows
  // apart; fp8 pools [NB, Hkv, bs, D]: (block, kv head) runs are contiguous.
  const uint32_t RS = KV8 ? (uint32_t)RB : (uint32_t)Hkv * RB;
  const size_t head_off = KV8 ? ((size_t)g * RB << bs_shift) : (size_t)g * RB;
  const char *kbase = (const char *)a.k_cache + head_off;
  const char *vbase = (const char *)a.v_cache + head_off;
  const int c16 = lane & 15, q4 = lane >> 4;

  // Q^T fragments: B operand of S^T = K Q^T.  Lane: query row c16 of each
  // 16-row block, head_dim elements 32 ks + 8 q4 .. +8.
  uint4 qf[2][KS];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int i = i0 + nb * 16 + c16;
    const uint4 *src = (const uint4 *)((const char *)a.q + ((size_t)(q0 + min(i, n - 1)) * Hq + h) * ROWB);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint4 v = src[ks * 4 + q4];
      qf[nb][ks] = i < n ? v : uint4{0u, 0u, 0u, 0u};
    }
  }

  // Block ids of the four 16-key groups of the tile starting at kt0 (one
  // block for block_size 256), clamped into the table.  Loaded one tile ahead
  // of their use so the scalar-load latency hides behind a tile of compute.
  const int Wm1 = a.max_blocks_per_seq - 1;
  auto tile_blocks = [&](int kt0, int (&blk)[KG]) {
#pragma unroll
    for (int q = 0; q < KG; ++q) blk[q] = table[min((kt0 + 16 * q) >> bs_shift, Wm1)];
  };

  // Tile DMA: the 2 * NDMA instructions of a tile are issued by NI waves,
  // NPW each.  Instruction jj of a tensor fills tile rows jj*RPD .. +RPD,
  // all inside the tile's 16-row group (jj*RPD) / 16, whose start row sits at
  // a scalar base; the per-lane part of the address is fixed for the launch.
  // Rows past the piece end re-read a valid row of the tile, so masked keys
  // only ever see finite data.
  uint32_t dma_voff[NPW];
#pragma unroll
  for (int jw = 0; jw < NPW; ++jw) {
    const int j = w + jw * NI;
    const bool is_v = j >= NDMA;
    const int jj = is_v ? j - NDMA : j;
    const int row_in = jj * RPD + lane / NCH;
    const int p = lane % NCH;
    const int c = KV8 ? (is_v ? v_pos8<D>(p, row_in) : k_pos8<D>(p, row_in))
                      : (is_v ? v_pos<D>(p, row_in) : k_pos<D>(p, row_in));
    dma_voff[jw] = (uint32_t)(row_in & 15) * RS + (uint32_t)c * 16;
  }
  auto issue_tile = [&](int kt0, int buf, const int (&blk)[KG]) {
    if (w >= NI) return;
    const char *gk[KG], *gv[KG];
#pragma unroll
    for (int q = 0; q < KG; ++q) {
      const int kg = kt0 + 16 * q;
      const size_t rows = ((size_t)(uint32_t)blk[q] << bs_shift) * (KV8 ? Hkv : 1);
      const size_t off = (rows + (size_t)(kg & bs_mask)) * RS;
      gk[q] = kbase + off;
      gv[q] = vbase + off;
    }
    const bool edge_tile = kt0 + kKeys > kend;
#pragma unroll
    for (int jw = 0; jw < NPW; ++jw) {
      const int j = w + jw * NI;
      const bool is_v = j >= NDMA;
      const int jj = is_v ? j - NDMA : j;
      const int grp = (jj * RPD) >> 4;
      const char *base = is_v ? gv[grp] : gk[grp];
      uint32_t voff = dma_voff[jw];
      if (edge_tile) {
        const int row_in = jj * RPD + lane / NCH;
        if (kt0 + jj * RPD >= kend) {
          base = is_v ? gv[0] : gk[0];               // whole instruction past the end:
          voff = voff - (uint32_t)(row_in & 15) * RS; // re-read tile row 0
        } else if (kt0 + row_in >= kend) {
          voff = voff - (uint32_t)(row_in & 15) * RS + (uint32_t)((jj * RPD) & 15) * RS;
        }
      }
      dma16(lds_offset(&smem[buf][is_v][jj * 1024]), base, voff);
    }
  };

  const int ntiles = (kend - kbeg + kKeys - 1) / kKeys;
  // blk: block ids of the next tile to issue; blk2 (pairs): of the one after
  int blk[KG], blk2[KG];
  if constexpr (PAIRS) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      if (t < ntiles) {
        tile_blocks(kbeg + t * kKeys, blk);
        issue_tile(kbeg + t * kKeys, t, blk);
      }
    }
    if (ntiles > 2) tile_blocks(kbeg + 2 * kKeys, blk);     // the second pair
    if (ntiles > 3) tile_blocks(kbeg + 3 * kKeys, blk2);
  } else {
#pragma unroll
    for (int t = 0; t < NST - 1; ++t) {
      if (t < ntiles) {
        tile_blocks(kbeg + t * kKeys, blk);
        issue_tile(kbeg + t * kKeys, t, blk);
      }
    }
    if (ntiles > NST - 1) tile_blocks(kbeg + (NST - 1) * kKeys, blk);   // for tile NST - 1
  }

  float m[2] = {-INFINITY, -INFINITY};
  f32x4 o[DB][2];
  f32x4 ol[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};  // row sums (all 4 equal)
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db][0] = o[db][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  const uint4 kOnes = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};  // bf16 1.0 x 8

  // Per-lane LDS offsets, fixed for the launch.  K fragment (key block mb,
  // step ks): row 16 mb + c16, chunk 4 ks + q4, stored at chunk ^ (row & 15)
  // = chunk ^ c16; the key block adds 16 rows.  V^T fragment (head_dim block
  // db, key step kk): source row 4 q4 + c16 / 4 (+ 32 kk, + 16 for the upper
  // half), columns 16 db + 4 (c16 % 4) in the 32-byte pair db ^ (row & 7).
  // fp8 pools: K fragment (mb, ks) is 8 bytes of row 16 mb + c16 at chunk
  // 2 ks + q4 / 2, half q4 % 2.  V^T fragment (db, kk): lane c16 addresses
  // half c16 % 2 of chunk db of key row kr = 4 q4 + k (k = c16 / 2 < 4) or
  // 16 + 4 q4 + k - 4 (k >= 4), + 32 kk; the transposing read hands it
  // column 16 db + c16 of its group's eight rows, k-th byte from row k.
  int k_off[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    k_off[ks] = KV8 ? c16 * RB + k_pos8<D>(2 * ks + (q4 >> 1), c16) * 16 + (q4 & 1) * 8
                    : c16 * ROWB + k_pos<D>(ks * 4 + q4, c16) * 16;
  const int tr_row = 4 * q4 + (c16 >> 2);
  const int kr = (c16 >> 1) < 4 ? 4 * q4 + (c16 >> 1) : 12 + 4 * q4 + (c16 >> 1);
  int v_off[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
    v_off[db] = KV8 ? kr * RB + v_pos8<D>(db, kr) * 16 + (c16 & 1) * 8
                    : tr_row * ROWB + v_pos<D>(2 * db + ((c16 & 3) >> 1), tr_row) * 16 + (c16 & 1) * 8;

  for (int it = 0; it < ntiles; ++it) {
    const int kt0 = kbeg + it * kKeys;
    if constexpr (PAIRS) {
      if ((it & 1) == 0) {
        // the pair (it, it + 1) is the only one in flight: once this wave's
        // DMAs are done, the barrier publishes everyone's and retires all
        // reads of the pair before, whose buffers the next pair takes
        wait_vmcnt<0>();
        __syncthreads();
        if (it + 2 < ntiles) issue_tile(kt0 + 2 * kKeys, (it + 2) & 3, blk);
        if (it + 3 < ntiles) issue_tile(kt0 + 3 * kKeys, (it + 3) & 3, blk2);
        if (it + 4 < ntiles) tile_blocks(kt0 + 4 * kKeys, blk);    // consumed at the next pair
        if (it + 5 < ntiles) tile_blocks(kt0 + 5 * kKeys, blk2);
      }
    } else {
      // this wave's DMAs of tile it are done when at most those of the tiles
      // issued after it (up to NST - 2) are outstanding; the barrier then
      // publishes everyone's tile it and retires all reads of the stage that
      // tile it + NST - 1 is about to overwrite (it held tile it - 1).
      wait_vmcnt_steps<NPW, NST - 2>(min(NST - 2, ntiles - 1 - it));
      __syncthreads();
      if (it + NST - 1 < ntiles) {
        issue_tile(kt0 + (NST - 1) * kKeys, (it + NST - 1) % NST, blk);
        if (it + NST < ntiles) tile_blocks(kt0 + NST * kKeys, blk);   // consumed next iteration
      }
    }
    const char *Kt = smem[it % NST][0];
    const char *Vt = smem[it % NST][1];

    // ---- S^T = K Q^T: KG key blocks x 2 row blocks, 2 KG independent chains ----
    f32x4 s[KG][2];
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    auto kfrag = [&](int ks, int mb) __attribute__((always_inline)) {
      const char *p = Kt + k_off[ks] + mb * 16 * RB;
      if constexpr (KV8)
        return fp8x8_to_bf16(*(const uint2 *)p);
      else
        return *(const uint4 *)p;
    };
#pragma unroll
    for (int mb = 0; mb < KG; ++mb) {
      const uint4 kf = kfrag(0, mb);
      s[mb][0] = mfma_k32(kf, qf[0][0], zero4);
      s[mb][1] = mfma_k32(kf, qf[1][0], zero4);
    }
#pragma unroll
    for (int ks = 1; ks < KS; ++ks) {
#pragma unroll
      for (int mb = 0; mb < KG; ++mb) {
        const uint4 kf = kfrag(ks, mb);
        s[mb][0] = mfma_k32(kf, qf[0][ks], s[mb][0]);
        s[mb][1] = mfma_k32(kf, qf[1][ks], s[mb][1]);
      }
    }

    // ---- online softmax, exp2 domain, lazily moved max ----
    // lane holds S^T[key = kt0 + 16 mb + 4 q4 + e][row = 16 nb + c16].
    // Interior tiles (no mask) with a positive scale keep the raw scores and
    // fold the scale into one fma per weight; edge tiles (causal diagonal or
    // piece end) scale and mask explicitly.
    const bool edge = (kt0 + kKeys > kend) || (kt0 + kKeys - 1 > pos0);
    const bool plain = !edge && a.scale_log2 > 0.f;
    float mxs[2];
    if (plain) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        float t = max3(s[0][nb][0], s[0][nb][1], s[0][nb][2]);
        t = max3(t, s[0][nb][3], s[1][nb][0]);
        t = max3(t, s[1][nb][1], s[1][nb][2]);
        t = max3(t, s[1][nb][3], t);
#pragma unroll
        for (int mb = 2; mb < KG; mb += 2) {
          t = max3(t, s[mb][nb][0], s[mb][nb][1]);
          t = max3(t, s[mb][nb][2], s[mb][nb][3]);
          t = max3(t, s[mb + 1][nb][0], s[mb + 1][nb][1]);
          t = max3(t, s[mb + 1][nb][2], s[mb + 1][nb][3]);
        }
        mxs[nb] = t * a.scale_log2;
      }
    } else {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int prow = pos0 + nb * 16 + c16;
        float t = -INFINITY;
#pragma unroll
        for (int mb = 0; mb < KG; ++mb)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int key = kt0 + mb * 16 + q4 * 4 + e;
            const float x = (key < kend && key <= prow) ? s[mb][nb][e] * a.scale_log2 : -INFINITY;
            s[mb][nb][e] = x;
            t = fmaxf(t, x);
          }
        mxs[nb] = t;
      }
    }
    const bool grow = (mxs[0] > m[0] + kSlackP) || (mxs[1] > m[1] + kSlackP);
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        float mx = fmaxf(m[nb], mxs[nb]);
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float alpha = mx == -INFINITY ? 1.f : exp2_fast(m[nb] - mx);
        m[nb] = mx;
        ol[nb] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) o[db][nb] *= alpha;
      }
    }
    // P^T fragments (B operand of O^T = V^T P^T), one per (row block, 32-key
    // step): lane holds keys 16 (2 kk) + 4 q4 + e and 16 (2 kk + 1) + 4 q4 + e.
    uint4 pf[2][KK];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const float mm = m[nb] == -INFINITY ? 0.f : m[nb];
      const float c = plain ? a.scale_log2 : 1.f;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        uint32_t pk[4];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const f32x4 sv = s[2 * kk + half][nb];
          pk[2 * half] = pack_bf16(exp2_fast(fmaf(sv[0], c, -mm)), exp2_fast(fmaf(sv[1], c, -mm)));
          pk[2 * half + 1] = pack_bf16(exp2_fast(fmaf(sv[2], c, -mm)), exp2_fast(fmaf(sv[3], c, -mm)));
        }
        pf[nb][kk] = uint4{pk[0], pk[1], pk[2], pk[3]};
      }
    }

    // ---- O^T += V^T P^T, and the row sums l += ones P^T on the same unit ----
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        uint4 vf;
        if constexpr (KV8) {
          vf = fp8x8_to_bf16(read_tr8(Vt + v_off[db] + kk * 32 * RB));
        } else {
          const char *vp = Vt + v_off[db] + kk * 32 * ROWB;
          const uint2 lo = read_tr(vp);
          const uint2 hi = read_tr(vp + 16 * ROWB);
          vf = uint4{lo.x, lo.y, hi.x, hi.y};
        }
        o[db][0] = mfma_k32(vf, pf[0][kk], o[db][0]);
        o[db][1] = mfma_k32(vf, pf[1][kk], o[db][1]);
      }
      ol[0] = mfma_k32(kOnes, pf[0][kk], ol[0]);
      ol[1] = mfma_k32(kOnes, pf[1][kk], ol[1]);
    }
  }

  // ---- normalise and write: lane holds O^T[d = 16 db + 4 q4 + e][row = 16 nb + c16] ----
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const float l = ol[nb][0];
    const int i = i0 + nb * 16 + c16;
    if (i >= n) continue;
    const size_t row = (size_t)(q0 + i) * Hq + h;
    float inv = l != 0.f ? 1.f / l : 0.f;
    if constexpr (KV8) inv *= a.v_scale;
    if (a.o_part == nullptr) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const f32x4 v = o[db][nb] * inv;
        uint2 pk;
        pk.x = pack_bf16(v[0], v[1]);
        pk.y = pack_bf16(v[2], v[3]);
        *(uint2 *)(a.out + row * D + 16 * db + 4 * q4) = pk;
      }
    } else {
      // workspace rows are [sequence, query index < max_q_len, q head, piece]
      if (i >= a.max_q_len) continue;
      const size_t prow = (((size_t)b * a.max_q_len + i) * Hq + h) * a.num_splits + piece;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const f32x4 v = o[db][nb] * inv;
        *(uint2 *)(a.o_part + prow * D + 16 * db + 4 * q4) =
            uint2{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
      }
      if (q4 == 0) a.lse_part[prow] = l != 0.f ? m[nb] + log2_fast(l) : -INFINITY;
    }
  }
}

// Merge the key pieces of (query index, q head) rows.  Grid: y = sequence b,
// x = blocks of rows j = i * Hq + h of that sequence (i < max_q_len).  A row's
// pieces sit at workspace row (b * max_q_len + i) * Hq + h, so every load of
// the row (its first BATCH pieces and their log-sum-exps) is issued at once,
// together with the sequence's offsets and length, before the number of
// non-empty pieces is known: pieces past it lie inside the workspace and are
// dropped by a select.  Query i sits at position p = L_b - n_b + i and has
// floor(p / split_len) + 1 non-empty pieces.  LPR lanes share a row, each
// owning 8 columns (one 16-byte load per piece), and every lane weighs the
// pieces itself, so the merge needs no cross-lane traffic; more than BATCH
// pieces are folded in batches with a running maximum.
template <int D>
__global__ __launch_bounds__(256) void prefill_merge_kernel(PrefillArgs a) {
  constexpr int LPR = D / 8;       // lanes per row
  constexpr int RPB = 256 / LPR;   // rows per workgroup
  constexpr int BATCH = 8;         // pieces in flight per lane
  const int sub = threadIdx.x % LPR;
  const int b = blockIdx.y;
  const int Hq = a.num_q_heads, S = a.num_splits;
  const int j = blockIdx.x * RPB + threadIdx.x / LPR;
  const int i = j / Hq, h = j % Hq;
  const size_t row = ((size_t)b * a.max_q_len + min(i, a.max_q_len - 1)) * Hq + h;
  const uint4 *op = (const uint4 *)(a.o_part + row * S * D) + sub;
  const float *lp = a.lse_part + row * S;
  const auto *cu = as_const(a.cu_seqlens_q);
  const int c0 = cu[b], n = cu[b + 1] - c0;
  const int L = as_const(a.context_lens)[b];
  uint4 ov[BATCH];
  float ls[BATCH];
#pragma unroll
  for (int k = 0; k < BATCH; ++k) {
    ov[k] = k < S ? op[(size_t)k * (D / 8)] : uint4{0u, 0u, 0u, 0u};
    ls[k] = k < S ? lp[k] : -INFINITY;
  }
  if (i >= n || i >= a.max_q_len) return;
  const int ns = min(S, (L - n + i) / a.split_len + 1);

  float M = -INFINITY, den = 0.f, acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  // fold pieces s0 .. s0 + BATCH - 1 (those below ns) into (M, den, acc)
  auto fold = [&](int s0) {
    float mb = M;
#pragma unroll
    for (int k = 0; k < BATCH; ++k)
      if (s0 + k < ns) mb = fmaxf(mb, ls[k]);
    const float alpha = M == -INFINITY ? 0.f : exp2_fast(M - mb);
    den *= alpha;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= alpha;
    M = mb;
#pragma unroll
    for (int k = 0; k < BATCH; ++k) {
      if (s0 + k < ns) {
        const float wk = exp2_fast(ls[k] - mb);
        den += wk;
        const uint32_t u[4] = {ov[k].x, ov[k].y, ov[k].z, ov[k].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * e] += wk * bf16_lo(u[e]);
          acc[2 * e + 1] += wk * bf16_hi(u[e]);
        }
      }
    }
  };
  fold(0);
  for (int s0 = BATCH; s0 < ns; s0 += BATCH) {
#pragma unroll
    for (int k = 0; k < BATCH; ++k) {
      const int s = min(s0 + k, S - 1);
      ov[k] = op[(size_t)s * (D / 8)];
      ls[k] = lp[s];
    }
    fold(s0);
  }
  const float inv = 1.f / den;
  uint4 pk;
  pk.x = pack_bf16(acc[0] * inv, acc[1] * inv);
  pk.y = pack_bf16(acc[2] * inv, acc[3] * inv);
  pk.z = pack_bf16(acc[4] * inv, acc[5] * inv);
  pk.w = pack_bf16(acc[6] * inv, acc[7] * inv);
  *((uint4 *)(a.out + ((size_t)(c0 + i) * Hq + h) * D) + sub) = pk;
}

template <int D, int G>
hipError_t launch_prefill_dg(const PrefillArgs &a, hipStream_t stream) {
  dim3 grid((a.max_q_len + kQRows - 1) / kQRows, a.num_kv_heads * a.num_splits, a.num_seqs);
  if (a.kv_fp8)
    hipLaunchKernelGGL((prefill_kernel<D, G, true>), grid, dim3(64 * G), 0, stream, a);
  else
    hipLaunchKernelGGL((prefill_kernel<D, G, false>), grid, dim3(64 * G), 0, stream, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_prefill_d(const PrefillArgs &a, int group, hipStream_t stream) {
  switch (group) {
    case 1: return launch_prefill_dg<D, 1>(a, stream);
    case 2: return launch_prefill_dg<D, 2>(a, stream);
    case 3: return launch_prefill_dg<D, 3>(a, stream);
    case 4: return launch_prefill_dg<D, 4>(a, stream);
    case 5: return launch_prefill_dg<D, 5>(a, stream);
    case 6: return launch_prefill_dg<D, 6>(a, stream);
    case 7: return launch_prefill_dg<D, 7>(a, stream);
    case 8: return launch_prefill_dg<D, 8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs &a, int head_dim, int group, hipStream_t stream) {
  if (head_dim == 128) return launch_prefill_d<128>(a, group, stream);
  if (head_dim == 64) return launch_prefill_d<64>(a, group, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_prefill_merge(const PrefillArgs &a, int head_dim, hipStream_t stream) {
  const int rows = a.max_q_len * a.num_q_heads;   // per sequence
  const int rpb = 256 / (head_dim / 8);
  dim3 grid((rows + rpb - 1) / rpb, a.num_seqs);
  if (head_dim == 128)
    hipLaunchKernelGGL(prefill_merge_kernel<128>, grid, dim3(256), 0, stream, a);
  else if (head_dim == 64)
    hipLaunchKernelGGL(prefill_merge_kernel<64>, grid, dim3(256), 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pa
