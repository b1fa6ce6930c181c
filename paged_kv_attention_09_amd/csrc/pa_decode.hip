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
//    NSTAGE chunks deep per wave.  The 16-byte positions of each row are
//    XOR-swizzled by row so both read patterns below are bank-conflict free.
//  * Scores: 4 lanes per token, each lane dots a quarter of the row against
//    the G query rows of the group with v_dot2c_f32_bf16 (q kept in VGPRs as
//    bf16 pairs), then a 2-step DPP quad sum.  This reads K once for all G
//    heads sharing the kv head.
//  * Online softmax per head in the exp2 domain: the chunk max over the 16
//    tokens (DPP row rotations + 4 readlanes) updates the running max m; the
//    weights exp2(x - m) are rounded to bf16 and parked in LDS.
//  * P.V: every lane owns 2 of the head_dim columns (1 for head_dim 64,
//    with two token halves) and walks the chunk's tokens in pairs: two bf16
//    V values of adjacent tokens are paired with a byte permute and one
//    v_dot2c per head accumulates both tokens into fp32.
//  * The 4 waves' (m, l, acc) are merged through LDS; the workgroup writes
//    either the final bf16 row (one piece) or an fp32 partial plus its
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
constexpr float kSlack = 8.f;  // log2 headroom before the running max moves

template <int D>
__device__ __forceinline__ int row_swizzle(int r) {
  return (r * 4) & (D / 8 - 1);
}

template <int D, int G, int NSTAGE>
struct DecodeLayout {
  static constexpr int ROWB = D * 2;                 // bytes of one token row (one kv head)
  static constexpr int NPOS = D / 8;                 // 16-byte positions per row
  static constexpr int CHB = kChunk * ROWB;          // bytes of one chunk of K (or V)
  static constexpr int NDMA = CHB / 1024;            // DMA instructions per tensor per chunk
  static constexpr int STB = 2 * CHB;                // one stage: K chunk then V chunk
  static constexpr int QB = ((G * ROWB + 1023) / 1024) * 1024;
  static constexpr int NQDMA = QB / 1024;
  static constexpr int PB = ((G * kChunk * 2 + 15) / 16) * 16;  // bf16 weights of a chunk
  static constexpr int WAVE_LDS = NSTAGE * STB + QB + PB;
  static constexpr int KPL = NPOS / 4;               // 16-byte K pieces per lane per token
  static constexpr int HALVES = 128 / D;             // token halves in the P.V layout
  static constexpr int PAIRS = kChunk / 2 / HALVES;  // token pairs per lane per chunk
  static_assert(WAVE_LDS % 16 == 0, "alignment");
  static_assert(2 * G + G * D <= (NSTAGE * STB) / 4, "merge scratch fits in the stages");
};

template <int D, int G, int NSTAGE>
__global__ __launch_bounds__(256, 2) void decode_split_kernel(DecodeArgs a) {
  using Lay = DecodeLayout<D, G, NSTAGE>;
  constexpr int ROWB = Lay::ROWB, NPOS = Lay::NPOS, CHB = Lay::CHB, NDMA = Lay::NDMA;
  constexpr int STB = Lay::STB, KPL = Lay::KPL, PAIRS = Lay::PAIRS;
  __shared__ __attribute__((aligned(1024))) char smem[kWaves * Lay::WAVE_LDS];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // Grid: x = (sequence, kv head), y = piece.  Workgroups dispatch in id
  // order and round-robin over the 8 XCDs, so every sequence's first piece
  // (never empty) goes out first and pieces of one index spread over all
  // XCDs instead of piling one piece index onto one XCD.
  const int g = blockIdx.x % a.num_kv_heads, b = blockIdx.x / a.num_kv_heads;
  const int split = blockIdx.y;
  const int Hq = a.num_q_heads;
  const int t0 = split * a.split_len;
  const size_t head0 = (size_t)b * Hq + (size_t)g * G;  // first q head of the group
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
      for (int i = threadIdx.x; i < G * D; i += 256) a.out[head0 * D + i] = 0;
    }
    return;
  }
  const int t1 = min(t0 + a.split_len, L);
  const int nck = (t1 - t0 + kChunk - 1) / kChunk;
  const int n_my = nck > wave ? (nck - wave + kWaves - 1) / kWaves : 0;

  char *my = smem + wave * Lay::WAVE_LDS;
  char *qlds = my + NSTAGE * STB;
  char *plds = qlds + Lay::QB;
  const uint32_t my_off = lds_offset(my);
  const uint32_t q_off = lds_offset(qlds);

  const uint32_t RS = (uint32_t)a.num_kv_heads * ROWB;  // bytes between token rows
  const char *kbase = (const char *)a.k_cache + (size_t)g * ROWB;
  const char *vbase = (const char *)a.v_cache + (size_t)g * ROWB;

  // Fused append: the wave that owns the sequence's last token writes the new
  // K/V row of this kv head to that token's slot, and waits for the stores to
  // complete before it issues any load of the chunk holding the row.  Only
  // this wave reads that row in this launch.
  if (a.new_k != nullptr && t1 == L && wave == (nck - 1) % kWaves) {
    const int tl = L - 1;
    const size_t row = ((size_t)(uint32_t)table[tl >> bs_shift] << bs_shift) + (tl & bs_mask);
    const size_t src = ((size_t)b * a.num_kv_heads + g) * ROWB;
    if (lane < 2 * NPOS) {
      const int c = lane % NPOS;
      const bool is_v = lane >= NPOS;
      const char *from = (const char *)(is_v ? a.new_v : a.new_k) + src + c * 16;
      char *to = (char *)(is_v ? vbase : kbase) + row * RS + c * 16;
      *(uint4 *)to = *(const uint4 *)from;
    }
    wait_vmcnt<0>();
  }

  // Per-lane DMA geometry: instruction j moves rows j*(1024/ROWB) + lane/NPOS.
  uint32_t dma_voff[NDMA], dma_pos[NDMA];
  int dma_row[NDMA];
#pragma unroll
  for (int j = 0; j < NDMA; ++j) {
    const int r = j * (1024 / ROWB) + lane / NPOS;
    const int p = lane % NPOS;
    const int c = p ^ row_swizzle<D>(r);
    dma_row[j] = r;
    dma_pos[j] = (uint32_t)c * 16;
    dma_voff[j] = (uint32_t)r * RS + (uint32_t)c * 16;
  }

  auto issue_chunk = [&](int ci, int stage, int blk) {
    const int tc = t0 + ci * kChunk;
    const size_t row0 = ((size_t)(uint32_t)blk << bs_shift) + (size_t)(tc & bs_mask);
    const char *kb = kbase + row0 * RS;
    const char *vb = vbase + row0 * RS;
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
      dma16(st + CHB + j * 1024, vb, vo);
    }
  };

  float m[G], l_lane[G], acc[G][2];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l_lane[h] = 0.f;
    acc[h][0] = acc[h][1] = 0.f;
  }

  if (n_my > 0) {
    // q rows of the group -> LDS (clamped lanes re-read the last 16 bytes).
    {
      const char *qsrc = (const char *)a.q + head0 * ROWB;
#pragma unroll
      for (int j = 0; j < Lay::NQDMA; ++j) {
        uint32_t o = (uint32_t)(j * 1024 + lane * 16);
        o = o < (uint32_t)(G * ROWB) ? o : (uint32_t)(G * ROWB - 16);
        dma16(q_off + j * 1024, qsrc, o);
      }
    }
#pragma unroll
    for (int s = 0; s < NSTAGE; ++s)
      if (s < n_my) issue_chunk(wave + kWaves * s, s, blk_first[s]);

    const int r = lane >> 2, u = lane & 3;
    const int swr = row_swizzle<D>(r);
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
      // ---- online softmax, exp2 domain, lazily rescaled ----
      // The running max m only moves when some score of the chunk exceeds it
      // by more than kSlack (one wave ballot decides); otherwise the weights
      // exp2(x - m) <= 2^kSlack stay well inside fp32/bf16 range and no
      // cross-lane max or rescale is needed.  The result is the same up to
      // rounding: numerator and denominator share the factor 2^-m.
      const bool valid = tc + r < t1;
      float x[G];
      bool grow = false;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        x[h] = valid ? quad_sum(s[h]) * a.scale_log2 : -INFINITY;
        grow |= x[h] > m[h] + kSlack;
      }
      if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float m_new = fmaxf(m[h], max_over_quads(x[h]));
          const float alpha = exp2_fast(m[h] - m_new);
          m[h] = m_new;
          l_lane[h] *= alpha;
          acc[h][0] *= alpha;
          acc[h][1] *= alpha;
        }
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const uint32_t pk = pack_bf16(exp2_fast(x[h] - m[h]), 0.f);
        l_lane[h] += bf16_lo(pk);
        // the 4 lanes of a token hold the same weight and all store it
        *(u16_alias *)(plds + h * (kChunk * 2) + r * 2) = (uint16_t)pk;
      }

      // ---- P.V: lanes own head_dim columns, tokens in pairs ----
      const char *vst = st + CHB;
#pragma unroll
      for (int jj = 0; jj < PAIRS; ++jj) {
        const int j = half * PAIRS + jj;
        const int ta = 2 * j, tb = 2 * j + 1;
        const uint32_t va = *(const uint32_t *)(vst + ta * ROWB + ((v_c ^ row_swizzle<D>(ta)) * 16) + v_in_chunk);
        const uint32_t vb = *(const uint32_t *)(vst + tb * ROWB + ((v_c ^ row_swizzle<D>(tb)) * 16) + v_in_chunk);
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

  // ---- merge the 4 waves through LDS ----
  float lsum[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    lsum[h] = sum_over_quads(l_lane[h]);
    if constexpr (D == 64) {
      acc[h][0] += __shfl_xor(acc[h][0], 32);
      acc[h][1] += __shfl_xor(acc[h][1], 32);
    }
  }
  float *mrg = (float *)my;  // [m: G][l: G][acc: G][D]
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      mrg[h] = m[h];
      mrg[G + h] = lsum[h];
    }
  }
  {
    const int dl = (D == 128) ? lane : (lane & 31);
    if (D == 128 || lane < 32) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float2 v2 = {acc[h][0], acc[h][1]};
        *(float2 *)(mrg + 2 * G + h * D + 2 * dl) = v2;
      }
    }
  }
  __syncthreads();

  const bool direct = a.o_part == nullptr;
  for (int idx = threadIdx.x; idx < G * D; idx += 256) {
    const int h = idx / D;
    float mw[kWaves];
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      mw[w] = ((const float *)(smem + w * Lay::WAVE_LDS))[h];
      M = fmaxf(M, mw[w]);
    }
    float den = 0.f, num = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float *mw_base = (const float *)(smem + w * Lay::WAVE_LDS);
        const float e = exp2_fast(mw[w] - M);
        den += e * mw_base[G + h];
        num += e * mw_base[2 * G + idx];
      }
    }
    // den is 0 only when no wave saw a token (empty sequence); a NaN read from
    // the cache propagates to the output.
    const float o = den != 0.f ? num / den : 0.f;
    if (direct) {
      a.out[head0 * D + idx] = (uint16_t)pack_bf16(o, 0.f);
    } else {
      const size_t row = (head0 + h) * a.num_splits + split;
      a.o_part[row * D + (idx % D)] = o;
      if (idx % D == 0) a.lse_part[row] = den != 0.f ? M + log2_fast(den) : -INFINITY;
    }
  }
}

// Merge the pieces of one (sequence, q head) row; one 256-thread workgroup
// per row.  Thread t reads lse of piece t; the workgroup max and the weights
// 2^(lse_s - M) go through LDS.  For the weighted sum, thread t owns float4
// column group t % (D/4) and pieces s = t / (D/4) (mod 256 / (D/4)); all of
// its piece loads are issued before the weights are known, so the row costs
// one memory round trip rather than one per piece.
template <int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeArgs a) {
  constexpr int NV = D / 4;        // float4 column groups per row
  constexpr int SG = 256 / NV;     // piece groups
  constexpr int BATCH = 8;         // piece loads in flight per thread
  __shared__ float w_lds[256];
  __shared__ float red_max[4], red_sum[4];
  __shared__ float4 red[SG][NV];
  const int h = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int L = as_const(a.context_lens)[b];
  const int S = a.num_splits;
  const size_t row = (size_t)b * a.num_q_heads + h;
  uint16_t *out = a.out + row * D;
  if (L <= 0) {
    if (tid < D) out[tid] = 0;
    return;
  }
  const int ns = min(S, (L + a.split_len - 1) / a.split_len);
  const int v = tid % NV, sg = tid / NV;
  const float4 *op = (const float4 *)(a.o_part + row * (size_t)S * D) + v;

  float4 ov[BATCH];
#pragma unroll
  for (int k = 0; k < BATCH; ++k) {
    const int s = sg + k * SG;
    ov[k] = s < ns ? op[(size_t)s * NV] : float4{0.f, 0.f, 0.f, 0.f};
  }
  const float lse = tid < ns ? a.lse_part[row * S + tid] : -INFINITY;
  float M = wave_max(lse);
  if (lane == 0) red_max[wv] = M;
  __syncthreads();
  M = fmaxf(fmaxf(red_max[0], red_max[1]), fmaxf(red_max[2], red_max[3]));
  const float w = tid < ns ? exp2_fast(lse - M) : 0.f;
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
    const float wk = w_lds[min(sg + k * SG, 255)];
    acc.x += wk * ov[k].x; acc.y += wk * ov[k].y; acc.z += wk * ov[k].z; acc.w += wk * ov[k].w;
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
    const float inv = 1.f / den;
    uint2 pk;
    pk.x = pack_bf16(t.x * inv, t.y * inv);
    pk.y = pack_bf16(t.z * inv, t.w * inv);
    *(uint2 *)(out + 4 * tid) = pk;
  }
}

constexpr int kStages = 2;

template <int D, int G>
hipError_t launch_split_dg(const DecodeArgs &a, int num_seqs, hipStream_t stream) {
  dim3 grid(num_seqs * a.num_kv_heads, a.num_splits);
  hipLaunchKernelGGL((decode_split_kernel<D, G, kStages>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
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
  dim3 grid(a.num_q_heads, num_seqs);
  if (head_dim == 128)
    hipLaunchKernelGGL(decode_combine_kernel<128>, grid, dim3(256), 0, stream, a);
  else if (head_dim == 64)
    hipLaunchKernelGGL(decode_combine_kernel<64>, grid, dim3(256), 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pa
