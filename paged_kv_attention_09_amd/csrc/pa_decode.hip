// Split-KV paged decode for gfx950.
//
// What is computed: for every sequence b and q head h, attention of the one
// query row over the sequence's cached tokens, read through its block table
// (PagedAttention via block tables: psmarter/mini-infer summary, "How It
// Works"; the unified [B, 1] paged decode of the mini-infer docs, "Core
// Capabilities at a Glance" table).  Long contexts are cut into split_len
// pieces processed by separate workgroups and merged afterwards by their
// log-sum-exp (flash decoding / split-K: zingnex.cn mini-infer thread,
// feature list item 7; MiniInfer README, "Attention Backend" table).
//
// How (one workgroup = one (piece, kv head, sequence), 4 waves):
//  * Each wave owns every 4th 16-token chunk of the piece.  A chunk always
//    lies inside one physical block (block_size 16 or 256), so the block id
//    is a scalar load and each DMA instruction has a scalar base address.
//  * K and V rows of a chunk (16 x head_dim bf16 each) stream HBM -> LDS with
//    global_load_lds_dwordx4 (16 bytes per lane, no VGPRs held in flight),
//    two chunks deep per wave.  The 16-byte positions of each row are XOR
//    swizzled by row so the LDS reads of the compute path are bank-conflict
//    free.
//  * Online softmax per head in the exp2 domain with a lazily moved running
//    max: the max moves (exact cross-lane max and rescale) only when a score
//    exceeds it by more than kSlack; a wave ballot decides.  Weights are
//    rounded to bf16 before the weighted V sum, and the denominator adds the
//    same rounded weights.
//  * Two compute paths for the per-chunk products, chosen by the group size
//    G (q heads per kv head):
//    - vector path (G <= 2): 4 lanes per token dot a quarter of the K row
//      each against the G query rows with v_dot2c_f32_bf16 and a DPP quad
//      sum; each lane owns 2 head_dim columns (1 for head_dim 64) and pairs
//      the V values of adjacent tokens with a byte permute, one v_dot2c per
//      token pair and head.
//    - matrix path (G >= 3): the G heads are the columns of a 16x16 tile
//      (columns G..15 zero).  S^T = K Q^T on v_mfma_f32_16x16x32_bf16 leaves
//      lane l with head l % 16 and tokens 4 (l / 16) + i; the bf16 weights,
//      in place, are the B operand of O^T += V^T P^T on
//      v_mfma_f32_16x16x16_bf16, with V^T read by ds_read_b64_tr_b16.  A
//      head's statistics and output column share lanes, so a rescale is
//      lane-local.  On the vector path the loop's ALU work grows with G and
//      at G = 6..7 it, not the memory system, set the pace.
//  * Several query tokens per sequence (the verify step of speculative
//    decoding): the matrix path's tile columns become (query token, head)
//    rows, one or two tiles, with query token j masking keys past
//    L - q_len + j; every staged chunk serves all of them.
//  * fp8 pools (e4m3 codes, head-major [NB, Hkv, bs, D]): the chunks stage
//    one byte per element; K fragments widen to bf16 in registers, and V^T
//    fragments come from the code chunk by an 8-bit transposing read and
//    widen in registers too; k_scale is folded into the score scale and
//    v_scale into the output.
//  * The 4 waves' (m, l, O) are merged through LDS; the workgroup writes
//    either the final bf16 rows (one piece) or fp32 partials plus their
//    base-2 log-sum-exp for the combine kernel.
//  * Tokens past the piece end are masked to -inf before the max; their DMA
//    lanes re-read the chunk's first row, so every load stays inside blocks
//    the table references and the masked lanes only ever see finite data.
#include "pa_device.hpp"
#include "pa_kernels.hpp"

namespace pa {

namespace {

constexpr int kWaves = 4;
constexpr int kChunk = 16;     // tokens per wave step
constexpr int kStages = 2;     // chunks in flight per wave
constexpr int kStages8 = 2;    // the same for fp8 pools (3 or 4 measured slower)
constexpr float kSlack = 8.f;  // log2 headroom before the running max moves
constexpr int kMaxVectorGroup = 2;

// LDS position of 16-byte chunk c of row r is c ^ row_swizzle(r).
//  vector path: lanes 4r..4r+3 read row r at positions u + 4k, so rows are
//    shifted by 4 positions each;
//  matrix path: 16 lanes read one position of rows 0..15, and the transposed
//    V reads take 8 rows x 2 adjacent positions per 32 lanes; a rotation of
//    the row index over the position bits serves both (for head_dim 64 two
//    rows share a 256-byte bank line, so the row pair index is rotated).
template <int D, bool MF>
__device__ __forceinline__ int row_swizzle(int r) {
  if constexpr (!MF) {
    return (r * 4) & (D / 8 - 1);
  } else if constexpr (D == 128) {
    return ((r << 1) | (r >> 3)) & 15;
  } else {
    const int s = r >> 1;
    return ((s << 1) | (s >> 2)) & 7;
  }
}

// fp8 pools: LDS position of 16-byte chunk c of stored row r (D bytes) is
// c ^ row_swizzle8(r).  Lanes of a K fragment read 8 bytes of rows 0..15 at
// one position; rows sharing a 256-byte bank line get distinct positions.
template <int D>
__device__ __forceinline__ int row_swizzle8(int r) {
  return (r >> (D == 128 ? 1 : 2)) & (D / 16 - 1);
}

template <int D>
struct DecodeGeom {
  static constexpr int ROWB = D * 2;                 // bytes of one token row (one kv head)
  static constexpr int NPOS = D / 8;                 // 16-byte positions per row
  static constexpr int CHB = kChunk * ROWB;          // bytes of one chunk of K (or V)
  static constexpr int NDMA = CHB / 1024;            // DMA instructions per tensor per chunk
  static constexpr int STB = 2 * CHB;                // one stage: K chunk then V chunk
  static constexpr int KS = D / 32;                  // matrix path: 16x16x32 steps over head_dim
  static constexpr int DB = D / 16;                  // matrix path: 16-column blocks of head_dim
  static constexpr int KPL = NPOS / 4;               // vector path: K pieces per lane per token
  static constexpr int HALVES = 128 / D;             // vector path: token halves in P.V
  static constexpr int PAIRS = kChunk / 2 / HALVES;  // vector path: token pairs per lane
  static constexpr int MS = D + 4;                   // merge scratch: floats per O row
};

// Per-wave LDS of the split kernel.  One query token: the DMA stages, the G
// q rows (staged by DMA, read once into registers) and, on the vector path,
// the bf16 weights of a chunk.  Several query tokens: the DMA stages only (the
// q rows go straight to registers).  The four-wave merge reuses the same
// bytes, in passes of at most `pass_rows` rows: m and l of the pass's rows,
// then its O rows; decode_merge_fits checks that they fit.
template <int D>
constexpr int decode_wave_lds(int q_rows, bool vector_path) {
  using Ge = DecodeGeom<D>;
  return kStages * Ge::STB + (q_rows * Ge::ROWB + 1023) / 1024 * 1024 +
         (vector_path ? (q_rows * kChunk * 2 + 15) / 16 * 16 : 0);
}
template <int D>
constexpr bool decode_merge_fits(int pass_rows, int wave_lds) {
  return (((2 * pass_rows + 3) & ~3) + pass_rows * DecodeGeom<D>::MS) * 4 <= wave_lds;
}
static_assert(decode_merge_fits<128>(8, decode_wave_lds<128>(1, false)) &&
                  decode_merge_fits<64>(8, decode_wave_lds<64>(1, false)) &&
                  decode_merge_fits<128>(16, decode_wave_lds<128>(0, false)) &&
                  decode_merge_fits<64>(16, decode_wave_lds<64>(0, false)) &&
                  decode_merge_fits<128>(kMaxVectorGroup, decode_wave_lds<128>(1, true)) &&
                  decode_merge_fits<64>(kMaxVectorGroup, decode_wave_lds<64>(1, true)),
              "merge scratch fits in the wave's LDS");

// MF selects the matrix path; NT is its number of 16-column tiles, which
// hold the G * q_len query rows (column c = query token c / G, head c % G).
// MULTI: q_len comes from the arguments, the q rows go straight to
// registers and the merge runs in passes of 16 rows; without it q_len is 1.
// The vector path handles one query token and NT = 1.
// KV8: the pools hold fp8 (e4m3) codes; the matrix path converts K fragments
// to bf16 in registers and each chunk's V into a bf16 LDS buffer, and the
// per-tensor scales fold into the score scale (K) and the output (V).
template <int D, int G, bool MF, int NT, bool MULTI, bool KV8>
__global__ __launch_bounds__(256, 2) void decode_split_kernel(DecodeArgs a) {
  static_assert(!KV8 || MF, "fp8 pools: matrix path");
  using Ge = DecodeGeom<D>;
  constexpr int NSTAGE = KV8 ? kStages8 : kStages;
  // bf16 rows, as computed on (q, the V^T reads, the merge)
  constexpr int ROWB = Ge::ROWB, CHB = Ge::CHB, KS = Ge::KS, DB = Ge::DB, MS = Ge::MS;
  constexpr int KPL = Ge::KPL, PAIRS = Ge::PAIRS;
  // rows as stored in the pool and staged by DMA (1 byte per element for fp8)
  constexpr int RB = KV8 ? D : ROWB;
  constexpr int NP = RB / 16;                      // 16-byte positions per stored row
  constexpr int CHK = kChunk * RB;                 // bytes of one staged chunk of K (or V)
  constexpr int NDMA = CHK / 1024;                 // DMA instructions per tensor per chunk
  constexpr int STB = 2 * CHK;                     // one stage: K chunk then V chunk
  // fp8 pools, several query tokens: room for the 16-row four-wave merge,
  // which needs more than the stages
  constexpr int CVB = KV8 && MULTI ? CHB : 0;
  constexpr int RC = MULTI ? 16 : G;   // rows per merge pass
  constexpr int WAVE_LDS =
      KV8 ? NSTAGE * STB + CVB + (MULTI ? 0 : (G * ROWB + 1023) / 1024 * 1024)
          : decode_wave_lds<D>(MULTI ? 0 : G, !MF);
  static_assert(!KV8 || decode_merge_fits<D>(RC, WAVE_LDS), "merge scratch");
  __shared__ __attribute__((aligned(1024))) char smem[kWaves * WAVE_LDS];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // Grid: x = (sequence, kv head), y = piece.  Workgroups dispatch in id
  // order and round-robin over the 8 XCDs, so every sequence's first piece
  // (never empty) goes out first and pieces of one index spread over all
  // XCDs instead of piling one piece index onto one XCD.  When the
  // workgroups are more than the compute units but at most two per compute
  // unit (mirror_second), the upper half of the pieces takes the units in
  // reverse order: the second-slot workgroup a compute unit receives then
  // belongs to the mirrored unit, so in a batch ordered longest first a long
  // sequence's early pieces share compute units with a short sequence's late
  // (mostly empty) ones instead of its own.
  const int split = blockIdx.y;
  const int ux = (a.mirror_second && 2 * split >= a.num_splits)
                     ? (int)gridDim.x - 1 - (int)blockIdx.x
                     : (int)blockIdx.x;
  const int g = ux % a.num_kv_heads, b = ux / a.num_kv_heads;
  const int Hq = a.num_q_heads;
  const int QL = MULTI ? a.q_len : 1;
  const int R = G * QL;                                   // query rows of this workgroup
  const int t0 = split * a.split_len;
  const size_t seq_row0 = (size_t)b * QL * Hq;            // first output row of the sequence
  // output row of query row r (token r / G, head g G + r % G)
  auto out_row = [&](int r) { return seq_row0 + (size_t)(r / G) * Hq + (size_t)g * G + r % G; };
  const int bs_shift = a.bs_shift;
  const int bs_mask = (1 << bs_shift) - 1;
  const int Wm1 = a.max_blocks_per_seq - 1;
  const auto *table = as_const(a.block_tables + (size_t)b * a.max_blocks_per_seq);

  // The length and the block ids of this wave's first chunks are independent
  // scalar loads, so they are in flight together (table entries past the
  // sequence end are read but never used).
  const int L = as_const(a.context_lens)[b];
  int blk_first[NSTAGE];
#pragma unroll
  for (int s = 0; s < NSTAGE; ++s)
    blk_first[s] = table[min((t0 + (wave + kWaves * s) * kChunk) >> bs_shift, Wm1)];

  if (t0 >= L) {
    // Nothing to read.  Only an empty sequence (L = 0) reaches this with
    // split 0; writing the output directly (one piece) this workgroup owns
    // the rows and writes zeros.  The merge never reads an empty piece.
    if (split == 0 && a.o_part == nullptr) {
      for (int i = threadIdx.x; i < R * D; i += 256) a.out[out_row(i / D) * D + i % D] = 0;
    }
    return;
  }
  const int t1 = min(t0 + a.split_len, L);
  const int nck = (t1 - t0 + kChunk - 1) / kChunk;
  const int n_my = nck > wave ? (nck - wave + kWaves - 1) / kWaves : 0;

  constexpr int QB = MULTI ? 0 : (G * ROWB + 1023) / 1024 * 1024;
  char *my = smem + wave * WAVE_LDS;
  char *qlds = my + NSTAGE * STB + CVB;
  char *plds = qlds + QB;  // vector path only
  const uint32_t my_off = lds_offset(my);
  const uint32_t q_off = lds_offset(qlds);

  // bf16 pools [NB, bs, Hkv, D]: token rows of one kv head are Hkv rows
  // apart.  fp8 pools [NB, Hkv, bs, D]: a (block, kv head) is one contiguous
  // run of bs rows.
  const uint32_t RS = KV8 ? (uint32_t)RB : (uint32_t)a.num_kv_heads * RB;  // between token rows
  const size_t head_off = KV8 ? ((size_t)g * RB << bs_shift) : (size_t)g * RB;
  const char *kbase = (const char *)a.k_cache + head_off;
  const char *vbase = (const char *)a.v_cache + head_off;
  // bytes from the pool start to row `off` of block `blk` (this kv head)
  auto row_offset = [&](int blk, int off) {
    const size_t rows = ((size_t)(uint32_t)blk << bs_shift);
    return KV8 ? (rows * a.num_kv_heads + (size_t)off) * RB : (rows + (size_t)off) * RS;
  };

  // Fused append (single query token only): the wave that owns the
  // sequence's last token writes the new K/V row of this kv head to that
  // token's slot (fp8 pools: quantised, 8 elements per lane), and waits for
  // the stores to complete before it issues any load of the chunk holding
  // the row.  Only this wave reads that row in this launch.
  if (!MULTI && a.new_k != nullptr && t1 == L && wave == (nck - 1) % kWaves) {
    constexpr int NPOS = Ge::NPOS;
    const int tl = L - 1;
    const size_t roff = row_offset(table[tl >> bs_shift], tl & bs_mask);
    const size_t src = ((size_t)b * a.num_kv_heads + g) * ROWB;
    if (lane < 2 * NPOS) {
      const int c = lane % NPOS;
      const bool is_v = lane >= NPOS;
      const uint4 x = *(const uint4 *)((const char *)(is_v ? a.new_v : a.new_k) + src + c * 16);
      char *to = (char *)(is_v ? vbase : kbase) + roff;
      if constexpr (KV8)
        *(uint2 *)(to + c * 8) = quantize8(x, is_v ? a.inv_v_scale : a.inv_k_scale);
      else
        *(uint4 *)(to + c * 16) = x;
    }
    wait_vmcnt<0>();
  }

  // Per-lane DMA geometry: instruction j moves rows j*(1024/RB) + lane/NP.
  uint32_t dma_voff[NDMA], dma_pos[NDMA];
  int dma_row[NDMA];
#pragma unroll
  for (int j = 0; j < NDMA; ++j) {
    const int r = j * (1024 / RB) + lane / NP;
    const int p = lane % NP;
    const int c = p ^ (KV8 ? row_swizzle8<D>(r) : row_swizzle<D, MF>(r));
    dma_row[j] = r;
    dma_pos[j] = (uint32_t)c * 16;
    dma_voff[j] = (uint32_t)r * RS + (uint32_t)c * 16;
  }

  auto issue_chunk = [&](int ci, int stage, int blk) {
    const int tc = t0 + ci * kChunk;
    const size_t boff = row_offset(blk, tc & bs_mask);
    const char *kb = kbase + boff;
    const char *vb = vbase + boff;
    const int nvalid = t1 - tc;
    const uint32_t st = my_off + stage * STB;
#pragma unroll
    for (int j = 0; j < NDMA; ++j) {
      const uint32_t vo = dma_row[j] < nvalid ? dma_voff[j] : dma_pos[j];
      dma16(st + j * 1024, kb, vo);
    }
#pragma unroll
    for (int j = 0; j < NDMA; ++j) {
      const uint32_t vo = dma_row[j] < nvalid ? dma_voff[j] : dma_pos[j];
      dma16(st + CHK + j * 1024, vb, vo);
    }
  };

  // Softmax state and accumulators.  Matrix path: in tile t, lane l holds
  // query row 16 t + l % 16 (m, partial l) and O^T[16 db + 4 qd + i][row].
  // Vector path: every lane holds all G heads' m and partial l, and head_dim
  // columns of acc.
  const int hh = lane & 15, qd = lane >> 4;
  float m_mf[NT], l_mf[NT];
  f32x4 o[MF ? NT : 1][MF ? DB : 1];
  float m_v[MF ? 1 : G], l_v[MF ? 1 : G], acc[MF ? 1 : G][2];
  if constexpr (MF) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      m_mf[t] = -INFINITY;
      l_mf[t] = 0.f;
#pragma unroll
      for (int d = 0; d < DB; ++d) o[t][d] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  } else {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      m_v[h] = -INFINITY;
      l_v[h] = 0.f;
      acc[h][0] = acc[h][1] = 0.f;
    }
  }

  // Q^T fragments of the matrix path: query row 16 t + hh (zero past the
  // last row), head_dim 32 kk + 8 qd .. + 7.
  uint4 qf[MF ? NT : 1][MF ? KS : 1];
  if (n_my > 0) {
    if constexpr (MULTI) {
      // straight to registers, issued before any DMA, so the first DMA wait
      // below also covers them
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int col = 16 * t + hh;
        const char *qrow = (const char *)a.q + out_row(min(col, R - 1)) * ROWB + qd * 16;
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
          const uint4 v = *(const uint4 *)(qrow + kk * 64);
          qf[t][kk] = col < R ? v : uint4{0u, 0u, 0u, 0u};
        }
      }
    } else {
      // the G query rows -> LDS: 16 bytes per lane (clamped lanes re-read the
      // last 16 bytes)
      const char *qsrc = (const char *)a.q + out_row(0) * ROWB;
#pragma unroll
      for (int j = 0; j < QB / 1024; ++j) {
        uint32_t off = (uint32_t)(j * 1024 + lane * 16);
        off = off < (uint32_t)(G * ROWB) ? off : (uint32_t)(G * ROWB - 16);
        dma16(q_off + j * 1024, qsrc, off);
      }
    }
#pragma unroll
    for (int s = 0; s < NSTAGE; ++s)
      if (s < n_my) issue_chunk(wave + kWaves * s, s, blk_first[s]);

    if constexpr (MF) {
      // LDS read offsets: K fragment kk of this lane is row hh, head_dim
      // 32 kk + 8 qd .. + 7; V^T fragment db is 8 bytes of row 4 qd + hh / 4
      // at head_dim 16 db + 4 (hh % 4).
      // fp8 pools: K fragment kk is 8 bytes of the stored row hh, at position
      // 2 kk + qd / 2, half qd % 2 (row_swizzle8 keeps these reads
      // conflict-free).  V^T fragment db comes from one 8-bit transposing
      // read: lane hh addresses half hh % 2 of position db of code row
      // 4 qd + (hh / 2) % 4 (lane pairs 4..7 repeat rows 0..3), and receives
      // head_dim 16 db + hh of rows 4 qd .. 4 qd + 3 as its bytes 0..3.
      uint32_t k_off[KS], v_off[DB];
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        if constexpr (KV8)
          k_off[kk] = (uint32_t)(hh * RB + (((2 * kk + (qd >> 1)) ^ row_swizzle8<D>(hh)) * 16) +
                                 (qd & 1) * 8);
        else
          k_off[kk] = (uint32_t)(hh * ROWB + (((4 * kk + qd) ^ row_swizzle<D, MF>(hh)) * 16));
      }
      if constexpr (KV8) {
        const int vr = 4 * qd + ((hh >> 1) & 3);
#pragma unroll
        for (int db = 0; db < DB; ++db)
          v_off[db] = (uint32_t)(CHK + vr * RB + ((db ^ row_swizzle8<D>(vr)) * 16) + (hh & 1) * 8);
      } else {
        const int vr = 4 * qd + (hh >> 2);
#pragma unroll
        for (int db = 0; db < DB; ++db)
          v_off[db] = (uint32_t)(CHB + vr * ROWB +
                                 (((2 * db + ((hh & 3) >> 1)) ^ row_swizzle<D, MF>(vr)) * 16) +
                                 (hh & 1) * 8);
      }
      // Per tile: is this lane's column a query row, and the last key its
      // query token may see (query token j sits at position L - q_len + j).
      bool colv[NT];
      int lim[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int col = 16 * t + hh;
        colv[t] = col < R;
        lim[t] = MULTI ? L - QL + col / G : L;
      }

      for (int i = 0; i < n_my; ++i) {
        wait_vmcnt_steps<2 * NDMA, NSTAGE - 1>(min(NSTAGE - 1, n_my - 1 - i));
        if constexpr (!MULTI) {
          if (i == 0) {
            const char *qrow = qlds + min(hh, G - 1) * ROWB + qd * 16;
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) {
              const uint4 v = *(const uint4 *)(qrow + kk * 64);
              qf[0][kk] = colv[0] ? v : uint4{0u, 0u, 0u, 0u};
            }
          }
        }
        const int ci = wave + kWaves * i;
        const int tc = t0 + ci * kChunk;
        const char *st = my + (i % NSTAGE) * STB;

        // ---- S^T = K Q^T: lane holds query row 16 t + hh, tokens 4 qd + e ----
        f32x4 sc[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) sc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
          uint4 kf;
          if constexpr (KV8)
            kf = fp8x8_to_bf16(*(const uint2 *)(st + k_off[kk]));
          else
            kf = *(const uint4 *)(st + k_off[kk]);
#pragma unroll
          for (int t = 0; t < NT; ++t) sc[t] = mfma_k32(kf, qf[t][kk], sc[t]);
        }

        // ---- online softmax, lazily rescaled (see the file comment) ----
        const int tok = tc + 4 * qd;
        float x[NT][4], cmax[NT];
        bool grow = false;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            x[t][e] = (tok + e < t1 && (!MULTI || tok + e <= lim[t])) ? sc[t][e] * a.scale_log2
                                                                      : -INFINITY;
          cmax[t] = fmaxf(fmaxf(x[t][0], x[t][1]), fmaxf(x[t][2], x[t][3]));
          grow |= colv[t] && cmax[t] > m_mf[t] + kSlack;
        }
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            float mx = fmaxf(m_mf[t], cmax[t]);
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float alpha = mx == -INFINITY ? 1.f : exp2_fast(m_mf[t] - mx);
            m_mf[t] = mx;
            l_mf[t] *= alpha;
#pragma unroll
            for (int d = 0; d < DB; ++d) o[t][d] *= alpha;
          }
        }
        uint2 pb[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const float mm = m_mf[t] == -INFINITY ? 0.f : m_mf[t];
          const uint32_t p01 = pack_bf16(exp2_fast(x[t][0] - mm), exp2_fast(x[t][1] - mm));
          const uint32_t p23 = pack_bf16(exp2_fast(x[t][2] - mm), exp2_fast(x[t][3] - mm));
          l_mf[t] += (bf16_lo(p01) + bf16_hi(p01)) + (bf16_lo(p23) + bf16_hi(p23));
          pb[t] = uint2{p01, p23};
        }

        // ---- O^T += V^T P^T: lane holds query row 16 t + hh, head_dim 16 db + 4 qd + i ----
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const uint2 vf = KV8 ? fp8x4_to_bf16(read_tr8(st + v_off[db]).x) : read_tr(st + v_off[db]);
#pragma unroll
          for (int t = 0; t < NT; ++t) o[t][db] = mfma_k16(vf, pb[t], o[t][db]);
        }

        if (i + NSTAGE < n_my) {
          const int cn = ci + kWaves * NSTAGE;
          issue_chunk(cn, i % NSTAGE, table[(t0 + cn * kChunk) >> bs_shift]);
        }
      }
    } else {
      const int r = lane >> 2, u = lane & 3;
      const int swr = row_swizzle<D, MF>(r);
      // P.V lane geometry
      const int half = (D == 128) ? 0 : (lane >> 5);
      const int dl = (D == 128) ? lane : (lane & 31);
      const uint32_t v_in_chunk = (uint32_t)(dl & 3) * 4;
      const int v_c = dl >> 2;

      uint4 qreg[G][KPL];
      for (int i = 0; i < n_my; ++i) {
        wait_vmcnt_steps<2 * NDMA, NSTAGE - 1>(min(NSTAGE - 1, n_my - 1 - i));
        if (i == 0) {
#pragma unroll
          for (int h = 0; h < G; ++h)
#pragma unroll
            for (int k = 0; k < KPL; ++k)
              qreg[h][k] = *(const uint4 *)(qlds + h * ROWB + (u + 4 * k) * 16);
        }
        const int ci = wave + kWaves * i;
        const int tc = t0 + ci * kChunk;
        const char *st = my + (i % NSTAGE) * STB;

        // ---- scores for the G heads, 4 lanes per token ----
        float s[G];
#pragma unroll
        for (int h = 0; h < G; ++h) s[h] = 0.f;
#pragma unroll
        for (int k = 0; k < KPL; ++k) {
          const int p = (u + 4 * k) ^ swr;
          const uint4 kv = *(const uint4 *)(st + r * ROWB + p * 16);
#pragma unroll
          for (int h = 0; h < G; ++h) {
            s[h] = dot2(qreg[h][k].x, kv.x, s[h]);
            s[h] = dot2(qreg[h][k].y, kv.y, s[h]);
            s[h] = dot2(qreg[h][k].z, kv.z, s[h]);
            s[h] = dot2(qreg[h][k].w, kv.w, s[h]);
          }
        }
        // ---- online softmax, lazily rescaled (see the file comment) ----
        const bool valid = tc + r < t1;
        float x[G];
        bool grow = false;
#pragma unroll
        for (int h = 0; h < G; ++h) {
          x[h] = valid ? quad_sum(s[h]) * a.scale_log2 : -INFINITY;
          grow |= x[h] > m_v[h] + kSlack;
        }
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
          for (int h = 0; h < G; ++h) {
            const float m_new = fmaxf(m_v[h], max_over_quads(x[h]));
            const float alpha = m_new == -INFINITY ? 1.f : exp2_fast(m_v[h] - m_new);
            m_v[h] = m_new;
            l_v[h] *= alpha;
            acc[h][0] *= alpha;
            acc[h][1] *= alpha;
          }
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float mm = m_v[h] == -INFINITY ? 0.f : m_v[h];
          const uint32_t pk = pack_bf16(exp2_fast(x[h] - mm), 0.f);
          l_v[h] += bf16_lo(pk);
          // the 4 lanes of a token hold the same weight and all store it
          *(u16_alias *)(plds + h * (kChunk * 2) + r * 2) = (uint16_t)pk;
        }

        // ---- P.V: lanes own head_dim columns, tokens in pairs ----
        const char *vst = st + CHB;
#pragma unroll
        for (int jj = 0; jj < PAIRS; ++jj) {
          const int j = half * PAIRS + jj;
          const int ta = 2 * j, tb = 2 * j + 1;
          const uint32_t va = *(const uint32_t *)(vst + ta * ROWB +
                                                  ((v_c ^ row_swizzle<D, MF>(ta)) * 16) + v_in_chunk);
          const uint32_t vb = *(const uint32_t *)(vst + tb * ROWB +
                                                  ((v_c ^ row_swizzle<D, MF>(tb)) * 16) + v_in_chunk);
          const uint32_t lo = lo_pair(va, vb), hi = hi_pair(va, vb);
#pragma unroll
          for (int h = 0; h < G; ++h) {
            const uint32_t pp = *(const u32_alias *)(plds + h * (kChunk * 2) + j * 4);
            acc[h][0] = dot2(pp, lo, acc[h][0]);
            acc[h][1] = dot2(pp, hi, acc[h][1]);
          }
        }

        if (i + NSTAGE < n_my) {
          const int cn = ci + kWaves * NSTAGE;
          issue_chunk(cn, i % NSTAGE, table[(t0 + cn * kChunk) >> bs_shift]);
        }
      }
    }
  }

  // ---- merge the 4 waves through LDS ----
  // Scratch per wave and pass: m[RC], l[RC], then from ACC0 one row of MS
  // floats per query row of the pass.  Each thread then finishes column
  // pairs of the pass's rows: all its LDS reads are issued before any
  // arithmetic (one LDS round trip), and a clamped index keeps the reads of
  // idle threads inside the table.
  constexpr int ACC0 = (2 * RC + 3) & ~3;
  constexpr int NIT = (RC * D / 2 + 255) / 256;
  float *mrg = (float *)my;
  const bool direct = a.o_part == nullptr;
  auto finish_rows = [&](int row_base, int rows) {
    const int npair = rows * D / 2;
    float mw[NIT][kWaves], lw[NIT][kWaves];
    float2 aw[NIT][kWaves];
#pragma unroll
    for (int k = 0; k < NIT; ++k) {
      const int pi = min((int)threadIdx.x + 256 * k, npair - 1);
      const int r = pi / (D / 2), c = 2 * (pi % (D / 2));
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float *wb = (const float *)(smem + w * WAVE_LDS);
        mw[k][w] = wb[r];
        lw[k][w] = wb[RC + r];
        aw[k][w] = *(const float2 *)(wb + ACC0 + r * MS + c);
      }
    }
#pragma unroll
    for (int k = 0; k < NIT; ++k) {
      const int pi = (int)threadIdx.x + 256 * k;
      if (pi >= npair) break;
      const int r = pi / (D / 2), c = 2 * (pi % (D / 2));
      float M = mw[k][0];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) M = fmaxf(M, mw[k][w]);
      float den = 0.f, n0 = 0.f, n1 = 0.f;
      if (M != -INFINITY) {
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
          const float e = exp2_fast(mw[k][w] - M);
          den += e * lw[k][w];
          n0 += e * aw[k][w].x;
          n1 += e * aw[k][w].y;
        }
      }
      // den is 0 only when no wave saw a key (an empty sequence, or a query
      // token whose keys all lie in other pieces); a NaN read from the cache
      // propagates to the output.
      float inv = den != 0.f ? 1.f / den : 0.f;
      if constexpr (KV8) inv *= a.v_scale;
      const size_t orow = out_row(row_base + r);
      if (direct) {
        *(uint32_t *)(a.out + orow * D + c) = pack_bf16(n0 * inv, n1 * inv);
      } else {
        const size_t row = orow * a.num_splits + split;
        *(float2 *)(a.o_part + row * D + c) = float2{n0 * inv, n1 * inv};
        if (c == 0) a.lse_part[row] = den != 0.f ? M + log2_fast(den) : -INFINITY;
      }
    }
  };

  if constexpr (MF) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      l_mf[t] += __shfl_xor(l_mf[t], 16);
      l_mf[t] += __shfl_xor(l_mf[t], 32);
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      // pass t: query rows 16 t .. 16 t + 15 (single token: the G heads)
      const int rows = min(RC, R - 16 * t);
      if (t > 0) __syncthreads();  // the previous pass has read the scratch
      if (hh < rows) {
        if (qd == 0) {
          mrg[hh] = m_mf[t];
          mrg[RC + hh] = l_mf[t];
        }
#pragma unroll
        for (int d = 0; d < DB; ++d) *(f32x4 *)(mrg + ACC0 + hh * MS + 16 * d + 4 * qd) = o[t][d];
      }
      __syncthreads();
      finish_rows(16 * t, rows);
    }
  } else {
    float lsum[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      lsum[h] = sum_over_quads(l_v[h]);
      if constexpr (D == 64) {
        acc[h][0] += __shfl_xor(acc[h][0], 32);
        acc[h][1] += __shfl_xor(acc[h][1], 32);
      }
    }
    if (lane == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        mrg[h] = m_v[h];
        mrg[G + h] = lsum[h];
      }
    }
    const int dl = (D == 128) ? lane : (lane & 31);
    if (D == 128 || lane < 32) {
#pragma unroll
      for (int h = 0; h < G; ++h)
        *(float2 *)(mrg + ACC0 + h * MS + 2 * dl) = float2{acc[h][0], acc[h][1]};
    }
    __syncthreads();
    finish_rows(0, G);
  }
}

// Merge the pieces of one (sequence, query token, q head) row when there are
// more than 64 pieces; one 256-thread workgroup per row.  Thread t reads lse of
// piece t; the workgroup max and the weights
// 2^(lse_s - M) go through LDS.  For the weighted sum, thread t owns float4
// column group t % (D/4) and pieces s = t / (D/4) (mod 256 / (D/4)).  Every
// load of the first batch (pieces, lse and the context length) is issued at
// once, before the number of non-empty pieces is known: rows of pieces past
// the sequence end lie inside the workspace and are dropped by a select, so
// the row costs one memory round trip.
template <int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeArgs a) {
  constexpr int NV = D / 4;        // float4 column groups per row
  constexpr int SG = 256 / NV;     // piece groups
  constexpr int BATCH = 8;         // piece loads in flight per thread
  __shared__ float w_lds[256];
  __shared__ float red_max[4], red_sum[4];
  __shared__ float4 red[SG][NV];
  const int h = blockIdx.x, b = blockIdx.y;  // h: (query token, q head) of the sequence
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int S = a.num_splits;
  const size_t row = (size_t)b * a.q_len * a.num_q_heads + h;
  const int v = tid % NV, sg = tid / NV;
  const float4 *op = (const float4 *)(a.o_part + row * (size_t)S * D) + v;

  const int L = as_const(a.context_lens)[b];
  float4 ov[BATCH];
#pragma unroll
  for (int k = 0; k < BATCH; ++k) {
    const int s = sg + k * SG;
    ov[k] = s < S ? op[(size_t)s * NV] : float4{0.f, 0.f, 0.f, 0.f};
  }
  const float lse_raw = tid < S ? a.lse_part[row * S + tid] : -INFINITY;

  uint16_t *out = a.out + row * D;
  if (L <= 0) {
    if (tid < D) out[tid] = 0;
    return;
  }
  const int ns = min(S, (L + a.split_len - 1) / a.split_len);
  const float lse = tid < ns ? lse_raw : -INFINITY;
  float M = wave_max(lse);
  if (lane == 0) red_max[wv] = M;
  __syncthreads();
  M = fmaxf(fmaxf(red_max[0], red_max[1]), fmaxf(red_max[2], red_max[3]));
  // M = -inf: no piece saw a key (a query token before position 0); the
  // weights are then 0, or NaN for a NaN partial, which must propagate.
  const float Mm = M == -INFINITY ? 0.f : M;
  const float w = tid < ns ? exp2_fast(lse - Mm) : 0.f;
  w_lds[tid] = w;
  float ws = w;
  ws += dpp<0xB1>(ws);
  ws += dpp<0x4E>(ws);
  ws = sum_over_quads(ws);
  if (lane == 0) red_sum[wv] = ws;
  __syncthreads();
  const float den = (red_sum[0] + red_sum[1]) + (red_sum[2] + red_sum[3]);

  float4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < BATCH; ++k) {
    const int s = sg + k * SG;
    if (s < ns) {
      const float wk = w_lds[s];
      acc.x += wk * ov[k].x; acc.y += wk * ov[k].y; acc.z += wk * ov[k].z; acc.w += wk * ov[k].w;
    }
  }
  for (int s0 = BATCH * SG; s0 < ns; s0 += BATCH * SG) {
#pragma unroll
    for (int k = 0; k < BATCH; ++k) {
      const int s = s0 + sg + k * SG;
      ov[k] = s < ns ? op[(size_t)s * NV] : float4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int k = 0; k < BATCH; ++k) {
      const float wk = w_lds[min(s0 + sg + k * SG, 255)];
      acc.x += wk * ov[k].x; acc.y += wk * ov[k].y; acc.z += wk * ov[k].z; acc.w += wk * ov[k].w;
    }
  }
  red[sg][v] = acc;
  __syncthreads();
  if (tid < NV) {
    float4 t = red[0][tid];
#pragma unroll
    for (int k = 1; k < SG; ++k) {
      t.x += red[k][tid].x; t.y += red[k][tid].y; t.z += red[k][tid].z; t.w += red[k][tid].w;
    }
    const float inv = den != 0.f ? 1.f / den : 0.f;
    uint2 pk;
    pk.x = pack_bf16(t.x * inv, t.y * inv);
    pk.y = pack_bf16(t.z * inv, t.w * inv);
    *(uint2 *)(out + 4 * tid) = pk;
  }
}

// The merge of at most 64 pieces, one 256-thread workgroup per row: every
// wave holds all the pieces' base-2 log-sum-exps (one per lane), so the
// maximum, the weights and their sum come from wave reductions; thread t owns
// float4 column group t / SG and pieces t % SG + SG k, so one column's pieces
// sit in SG consecutive lanes and sum by shuffles: no LDS and no barrier.  As
// in the kernel above, every load is issued before the number of non-empty
// pieces is known and pieces past it are dropped by a select.
template <int D>
__global__ __launch_bounds__(256) void decode_combine64_kernel(DecodeArgs a) {
  constexpr int NV = D / 4;          // float4 columns per row
  constexpr int SG = 256 / NV;       // lanes per column
  constexpr int BATCH = 64 / SG;     // pieces per lane
  const int h = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int S = a.num_splits;
  const size_t row = (size_t)b * a.q_len * a.num_q_heads + h;
  const int v = tid / SG, sg = tid % SG;
  const float4 *op = (const float4 *)(a.o_part + row * (size_t)S * D) + v;
  const int L = as_const(a.context_lens)[b];
  float4 ov[BATCH];
#pragma unroll
  for (int k = 0; k < BATCH; ++k) {
    const int s = sg + k * SG;
    ov[k] = s < S ? op[(size_t)s * NV] : float4{0.f, 0.f, 0.f, 0.f};
  }
  const float lse_raw = lane < S ? a.lse_part[row * S + lane] : -INFINITY;
  uint16_t *out = a.out + row * D;
  if (L <= 0) {
    if (tid < D) out[tid] = 0;
    return;
  }
  const int ns = min(S, (L + a.split_len - 1) / a.split_len);
  const float lse = lane < ns ? lse_raw : -INFINITY;
  const float M = wave_max(lse);
  const float Mm = M == -INFINITY ? 0.f : M;
  const float w = lane < ns ? exp2_fast(lse - Mm) : 0.f;
  const float den = wave_sum(w);
  float4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < BATCH; ++k) {
    const int s = sg + k * SG;
    const float wk = __shfl(w, s);
    if (s < ns) {
      acc.x += wk * ov[k].x; acc.y += wk * ov[k].y; acc.z += wk * ov[k].z; acc.w += wk * ov[k].w;
    }
  }
#pragma unroll
  for (int off = 1; off < SG; off <<= 1) {
    acc.x += __shfl_xor(acc.x, off);
    acc.y += __shfl_xor(acc.y, off);
    acc.z += __shfl_xor(acc.z, off);
    acc.w += __shfl_xor(acc.w, off);
  }
  if (sg == 0) {
    const float inv = den != 0.f ? 1.f / den : 0.f;
    uint2 pk;
    pk.x = pack_bf16(acc.x * inv, acc.y * inv);
    pk.y = pack_bf16(acc.z * inv, acc.w * inv);
    *(uint2 *)(out + 4 * v) = pk;
  }
}

template <int D, int G, bool MF, int NT, bool MULTI, bool KV8 = false>
hipError_t launch_split_variant(const DecodeArgs &a, int num_seqs, hipStream_t stream) {
  dim3 grid(num_seqs * a.num_kv_heads, a.num_splits);
  hipLaunchKernelGGL((decode_split_kernel<D, G, MF, NT, MULTI, KV8>), grid, dim3(256), 0, stream,
                     a);
  return hipGetLastError();
}

// Path choice: one query token with a group of at most kMaxVectorGroup heads
// takes the vector path, other single-token groups the matrix path with one
// tile; several query tokens take the matrix path with one tile per 16 rows.
// fp8 pools always take the matrix path.
template <int D, int G, bool KV8>
hipError_t launch_split_dgk(const DecodeArgs &a, int num_seqs, hipStream_t stream) {
  if (a.q_len == 1) {
    if constexpr (G <= kMaxVectorGroup && !KV8)
      return launch_split_variant<D, G, false, 1, false>(a, num_seqs, stream);
    else
      return launch_split_variant<D, G, true, 1, false, KV8>(a, num_seqs, stream);
  }
  const int rows = G * a.q_len;
  if (rows <= 16) return launch_split_variant<D, G, true, 1, true, KV8>(a, num_seqs, stream);
  if constexpr (G * kMaxQueryTokens > 16) {
    if (rows <= kMaxDecodeRows)
      return launch_split_variant<D, G, true, 2, true, KV8>(a, num_seqs, stream);
  }
  return hipErrorInvalidValue;
}

template <int D, int G>
hipError_t launch_split_dg(const DecodeArgs &a, int num_seqs, hipStream_t stream) {
  if (a.new_k != nullptr && a.q_len != 1) return hipErrorInvalidValue;
  if (a.kv_fp8) return launch_split_dgk<D, G, true>(a, num_seqs, stream);
  return launch_split_dgk<D, G, false>(a, num_seqs, stream);
}

template <int D>
hipError_t launch_split_d(const DecodeArgs &a, int group, int num_seqs, hipStream_t stream) {
  switch (group) {
    case 1: return launch_split_dg<D, 1>(a, num_seqs, stream);
    case 2: return launch_split_dg<D, 2>(a, num_seqs, stream);
    case 3: return launch_split_dg<D, 3>(a, num_seqs, stream);
    case 4: return launch_split_dg<D, 4>(a, num_seqs, stream);
    case 5: return launch_split_dg<D, 5>(a, num_seqs, stream);
    case 6: return launch_split_dg<D, 6>(a, num_seqs, stream);
    case 7: return launch_split_dg<D, 7>(a, num_seqs, stream);
    case 8: return launch_split_dg<D, 8>(a, num_seqs, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode_split(const DecodeArgs &a, int head_dim, int group, int num_seqs,
                               hipStream_t stream) {
  if (head_dim == 128) return launch_split_d<128>(a, group, num_seqs, stream);
  if (head_dim == 64) return launch_split_d<64>(a, group, num_seqs, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_decode_combine(const DecodeArgs &a, int head_dim, int num_seqs,
                                 hipStream_t stream) {
  dim3 grid(a.num_q_heads * a.q_len, num_seqs);
  const bool small = a.num_splits <= 64;
  if (head_dim == 128) {
    if (small)
      hipLaunchKernelGGL(decode_combine64_kernel<128>, grid, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL(decode_combine_kernel<128>, grid, dim3(256), 0, stream, a);
  } else if (head_dim == 64) {
    if (small)
      hipLaunchKernelGGL(decode_combine64_kernel<64>, grid, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL(decode_combine_kernel<64>, grid, dim3(256), 0, stream, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pa
