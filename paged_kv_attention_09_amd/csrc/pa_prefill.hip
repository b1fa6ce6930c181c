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
//  * Key tiles of 64 rows stream into LDS by global_load_lds_dwordx4,
//    double buffered.  K rows are stored with their 16-byte chunks XOR
//    swizzled by row, V rows with their 32-byte column pairs swizzled, so the
//    reads below hit distinct banks.
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
//    tiles that cross them.
#include "pa_device.hpp"
#include "pa_kernels.hpp"

namespace pa {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int kQRows = 32;   // query positions per workgroup (two 16-row MFMA blocks)
constexpr int kKeys = 64;    // keys per LDS tile
constexpr float kSlackP = 8.f;

__device__ __forceinline__ f32x4 mfma16(const uint4 &a, const uint4 &b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint2 read_tr(const char *p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4 *)(__attribute__((address_space(3))) void *)p);
  return __builtin_bit_cast(uint2, v);
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

template <int D, int G>
__global__ __launch_bounds__(64 * G) void prefill_kernel(PrefillArgs a) {
  using Lay = PrefillLayout<D>;
  constexpr int ROWB = Lay::ROWB, TILEB = Lay::TILEB, NDMA = Lay::NDMA, KS = Lay::KSTEPS;
  constexpr int DB = Lay::DBLK, RPD = Lay::ROWS_PER_DMA, NCH = Lay::NCH;
  __shared__ __attribute__((aligned(1024))) char smem[2][2][TILEB];  // [buffer][K, V]

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
  const uint32_t RS = (uint32_t)Hkv * ROWB;
  const char *kbase = (const char *)a.k_cache + (size_t)g * ROWB;
  const char *vbase = (const char *)a.v_cache + (size_t)g * ROWB;
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

  // Tile DMA: the 2 * NDMA instructions of a tile are spread over the waves.
  auto issue_tile = [&](int kt0, int buf) {
    for (int j = w; j < 2 * NDMA; j += G) {
      const bool is_v = j >= NDMA;
      const int jj = is_v ? j - NDMA : j;
      const int rfirst = kt0 + jj * RPD;                 // first key of this instruction
      const int row_in = jj * RPD + lane / NCH;          // tile row this lane fills
      const int p = lane % NCH;                          // stored 16-byte position
      const int c = is_v ? v_pos<D>(p, row_in) : k_pos<D>(p, row_in);
      int key = kt0 + row_in, kfirst = rfirst;
      if (rfirst >= kend) kfirst = kt0;                  // whole instruction past the end:
      if (key >= kend) key = kfirst;                     // re-read a valid row (finite data)
      const size_t row0 = ((size_t)(uint32_t)table[kfirst >> bs_shift] << bs_shift) +
                          (size_t)(kfirst & bs_mask);
      const uint32_t voff = (uint32_t)(key - kfirst) * RS + (uint32_t)c * 16;
      const char *base = (is_v ? vbase : kbase) + row0 * RS;
      dma16(lds_offset(&smem[buf][is_v][jj * 1024]), base, voff);
    }
  };

  const int ntiles = (kend - kbeg + kKeys - 1) / kKeys;
  issue_tile(kbeg, 0);

  float m[2] = {-INFINITY, -INFINITY};
  float lsum[2] = {0.f, 0.f};
  f32x4 o[DB][2];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db][0] = o[db][1] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int it = 0; it < ntiles; ++it) {
    wait_vmcnt<0>();
    __syncthreads();
    const int kt0 = kbeg + it * kKeys;
    if (it + 1 < ntiles) issue_tile(kt0 + kKeys, (it + 1) & 1);
    const char *Kt = smem[it & 1][0];
    const char *Vt = smem[it & 1][1];

    // ---- S^T = K Q^T: 4 key blocks x 2 row blocks ----
    f32x4 s[4][2];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      s[mb][0] = s[mb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int r = mb * 16 + c16;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint4 kf = *(const uint4 *)(Kt + r * ROWB + k_pos<D>(ks * 4 + q4, r) * 16);
        s[mb][0] = mfma16(kf, qf[0][ks], s[mb][0]);
        s[mb][1] = mfma16(kf, qf[1][ks], s[mb][1]);
      }
    }

    // ---- scale, masks, lazily rescaled online softmax ----
    // lane holds S^T[key = kt0 + 16 mb + 4 q4 + e][row = 16 nb + c16]
    const bool edge = (kt0 + kKeys > kend) || (kt0 + kKeys - 1 > pos0);
    bool grow = false;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int prow = pos0 + nb * 16 + c16;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float x = s[mb][nb][e] * a.scale_log2;
          if (edge) {
            const int key = kt0 + mb * 16 + q4 * 4 + e;
            x = (key < kend && key <= prow) ? x : -INFINITY;
          }
          s[mb][nb][e] = x;
          grow |= x > m[nb] + kSlackP;
        }
    }
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        float mx = m[nb];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
          for (int e = 0; e < 4; ++e) mx = fmaxf(mx, s[mb][nb][e]);
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float alpha = mx == -INFINITY ? 1.f : exp2_fast(m[nb] - mx);
        m[nb] = mx;
        lsum[nb] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) o[db][nb] *= alpha;
      }
    }
    // P^T fragments (B operand of O^T = V^T P^T), one per (row block, 32-key
    // step): lane holds keys 16 (2 kk) + 4 q4 + e and 16 (2 kk + 1) + 4 q4 + e.
    uint4 pf[2][2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const float mm = m[nb] == -INFINITY ? 0.f : m[nb];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        uint32_t pk[4];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const f32x4 sv = s[2 * kk + half][nb];
          pk[2 * half] = pack_bf16(exp2_fast(sv[0] - mm), exp2_fast(sv[1] - mm));
          pk[2 * half + 1] = pack_bf16(exp2_fast(sv[2] - mm), exp2_fast(sv[3] - mm));
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) lsum[nb] += bf16_lo(pk[t]) + bf16_hi(pk[t]);
        pf[nb][kk] = uint4{pk[0], pk[1], pk[2], pk[3]};
      }
    }

    // ---- O^T += V^T P^T: head_dim blocks x 2 row blocks x 2 key steps ----
    // V^T fragment lane (q4, c16): V[16 kb + 4 q4 + j][16 db + c16], j = 0..3,
    // for kb = 2 kk and 2 kk + 1, via transposing reads: source lane s of the
    // 16-lane group addresses row 4 q4 + s / 4, columns 16 db + 4 (s % 4).
    const int tr_row = 4 * q4 + (c16 >> 2);
    const int tr_col_chunk_lo = (c16 & 3) >> 1;   // which 16-byte half of the 32-byte pair
    const int tr_byte = (c16 & 1) * 8;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int r0 = 32 * kk + tr_row, r1 = r0 + 16;
        const int c = 2 * db + tr_col_chunk_lo;
        const uint2 lo = read_tr(Vt + r0 * ROWB + v_pos<D>(c, r0) * 16 + tr_byte);
        const uint2 hi = read_tr(Vt + r1 * ROWB + v_pos<D>(c, r1) * 16 + tr_byte);
        const uint4 vf = uint4{lo.x, lo.y, hi.x, hi.y};
        o[db][0] = mfma16(vf, pf[0][kk], o[db][0]);
        o[db][1] = mfma16(vf, pf[1][kk], o[db][1]);
      }
    }
  }

  // ---- normalise and write: lane holds O^T[d = 16 db + 4 q4 + e][row = 16 nb + c16] ----
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    float l = lsum[nb];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    const int i = i0 + nb * 16 + c16;
    if (i >= n) continue;
    const size_t row = (size_t)(q0 + i) * Hq + h;
    const float inv = l != 0.f ? 1.f / l : 0.f;
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
      const size_t prow = row * a.num_splits + piece;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const f32x4 v = o[db][nb] * inv;
        *(float4 *)(a.o_part + prow * D + 16 * db + 4 * q4) = float4{v[0], v[1], v[2], v[3]};
      }
      if (q4 == 0) a.lse_part[prow] = l != 0.f ? m[nb] + log2_fast(l) : -INFINITY;
    }
  }
}

// Merge the key pieces of one (query row, q head): row t of sequence b sits
// at position p = L_b - n_b + (t - cu[b]) and has floor(p / split_len) + 1
// non-empty pieces.  One 64-lane wave per output row.
template <int D>
__global__ __launch_bounds__(64) void prefill_merge_kernel(PrefillArgs a) {
  const int h = blockIdx.x, t = blockIdx.y;
  const int lane = threadIdx.x;
  const auto *cu = as_const(a.cu_seqlens_q);
  if (t >= cu[a.num_seqs]) return;   // the grid covers num_seqs * max_q_len rows
  int b = 0;
  while (b + 1 < a.num_seqs && cu[b + 1] <= t) ++b;
  const int n = cu[b + 1] - cu[b];
  const int p = as_const(a.context_lens)[b] - n + (t - cu[b]);
  const int S = a.num_splits;
  const int ns = min(S, p / a.split_len + 1);
  const size_t row = (size_t)t * a.num_q_heads + h;
  const float *lse = a.lse_part + row * S;
  constexpr int PER = D / 64;
  float M = -INFINITY;
  for (int s = lane; s < ns; s += 64) M = fmaxf(M, lse[s]);
  M = wave_max(M);
  float den = 0.f, acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  const float *op = a.o_part + row * (size_t)S * D + lane * PER;
  for (int s = 0; s < ns; ++s) {
    const float wgt = exp2_fast(lse[s] - M);
    den += wgt;
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] += wgt * op[(size_t)s * D + e];
  }
  const float inv = 1.f / den;
  uint16_t *out = a.out + row * D + lane * PER;
#pragma unroll
  for (int e = 0; e < PER; ++e) out[e] = (uint16_t)pack_bf16(acc[e] * inv, 0.f);
}

template <int D, int G>
hipError_t launch_prefill_dg(const PrefillArgs &a, hipStream_t stream) {
  dim3 grid((a.max_q_len + kQRows - 1) / kQRows, a.num_kv_heads * a.num_splits, a.num_seqs);
  hipLaunchKernelGGL((prefill_kernel<D, G>), grid, dim3(64 * G), 0, stream, a);
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

hipError_t launch_prefill_merge(const PrefillArgs &a, int head_dim, int total_q,
                                hipStream_t stream) {
  dim3 grid(a.num_q_heads, total_q);
  if (head_dim == 128)
    hipLaunchKernelGGL(prefill_merge_kernel<128>, grid, dim3(64), 0, stream, a);
  else if (head_dim == 64)
    hipLaunchKernelGGL(prefill_merge_kernel<64>, grid, dim3(64), 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pa
