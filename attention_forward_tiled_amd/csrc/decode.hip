// Split-KV decode and the log-sum-exp combine for gfx950.
//
// What is computed: one query row per (sequence, query head) against all of the
// sequence's keys, split along the key axis into partitions whose partial,
// softmax-weighted outputs are then merged (page "gfx942 unified attention, from
// the math up", section 8; a single query attends to every key, section 4). Each
// split runs the online-softmax recurrence of section 3 over its 64-key pages and
// leaves a normalised O_s and lse_s = ln(sum over the split of e^(s_j)); the combine
// weights the splits by e^(lse_s - max lse).
//
// How it is mapped onto CDNA4 (the split kernel streams K/V once from HBM and is
// bandwidth-bound, so the layout choices are about bytes in flight, not flops):
//   * One workgroup (4 waves) per (partition, KV head, sequence). The G query heads
//     that share the KV head are processed together, so every K/V byte is read once.
//   * Waves take whole pages round-robin inside the partition and keep their own
//     running (m, l, o); the four states are merged through LDS at the end.
//   * Per page, the wave issues all of its K and V loads up front (16-byte loads,
//     each wave instruction covering whole 256-byte rows for d = 128), then computes
//     S^T = K Q^T with v_mfma_f32_16x16x32 (Q padded to 16 columns, K loaded straight
//     into the A-operand layout), and accumulates P.V on the vector ALUs: V rows are
//     consumed in their natural layout, with P broadcast through a small per-wave LDS
//     buffer.
//   * Keys past the sequence length (NaN-poisoned page tails) load as zeros and their
//     scores are masked, so they never reach the output.
#include "common.hpp"
#include "kernels.hpp"

namespace attn {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

template <int D, typename T, int GT>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(const DecodeParams p) {
  constexpr int KS = D / 32;              // k-steps of S^T
  constexpr int CPR = D / 8;              // 16-byte chunks per key row
  constexpr int RPL = 64 / CPR;           // key rows covered by one wave-wide load
  constexpr int VL = kPage / RPL;         // V loads per lane per page
  __shared__ float p_lds[kWaves][kPage][GT];
  __shared__ float st_m[kWaves][GT], st_l[kWaves][GT];
  __shared__ float o_lds[kWaves][GT][D];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lr = lane & 15, lg = lane >> 4;
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int G = p.group;

  const int L = min(max(p.seqlens_k[b], 0), p.max_seqlen_k);
  const int start = split * p.part_tokens;
  const int end = min(start + p.part_tokens, L);
  const int64_t out_row0 = ((int64_t)b * p.hq + (int64_t)kvh * G) * p.num_splits + split;

  if (start >= end) {  // empty partition: O_s = 0, lse_s = -inf
    for (int i = tid; i < G * D; i += kThreads) {
      const int g = i / D, d = i % D;
      p.part_o[(out_row0 + (int64_t)g * p.num_splits) * D + d] = 0.f;
    }
    if (tid < G) p.part_lse[out_row0 + (int64_t)tid * p.num_splits] = -INFINITY;
    return;
  }

  // Q fragments (B operand): lane lr holds query head lr of the group (zero if lr >= G).
  u32x4 qf[KS];
  {
    const bool ok = lr < G;
    const uint16_t* qp = p.q + ((int64_t)b * p.hq + (int64_t)kvh * G + (ok ? lr : 0)) * D;
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = ok ? ldg16(qp + s * 32 + lg * 8) : u32x4{0, 0, 0, 0};
  }

  const int vrow = lane / CPR, vch = lane % CPR;  // this lane's V row offset / chunk
  float m = -INFINITY, lsum = 0.f;                 // S^T layout: query lr
  float acc[GT][8];                                // P.V layout: queries x 8 d of chunk vch
#pragma unroll
  for (int g = 0; g < GT; ++g)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[g][e] = 0.f;

  const int first_page = start / kPage;
  const int n_pages = (end - start + kPage - 1) / kPage;
  const int64_t row_stride = (int64_t)p.hkv * D;

  for (int pi = wave; pi < n_pages; pi += kWaves) {
    const int lp = first_page + pi;
    const int key0 = lp * kPage;
    const int pg = p.block_table[(int64_t)b * p.max_blocks + lp];
    const bool page_ok = pg >= 0 && pg < p.num_blocks;
    const int n_valid = page_ok ? min(kPage, end - key0) : 0;
    const int64_t base = (int64_t)(page_ok ? pg : 0) * kPage * row_stride + (int64_t)kvh * D;

    u32x4 kf[4][KS];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int row = kb * 16 + lr;
      const bool ok = row < n_valid;
#pragma unroll
      for (int s = 0; s < KS; ++s)
        kf[kb][s] = ok ? ldg16(p.k + base + row * row_stride + s * 32 + lg * 8) : u32x4{0, 0, 0, 0};
    }
    u32x4 vf[VL];
#pragma unroll
    for (int jj = 0; jj < VL; ++jj) {
      const int row = jj * RPL + vrow;
      vf[jj] = row < n_valid ? ldg16(p.v + base + row * row_stride + vch * 8) : u32x4{0, 0, 0, 0};
    }

    // S^T: lane holds query lr, keys kb*16 + 4*lg + i
    float x[4][4];
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      float4v s = {0, 0, 0, 0};
#pragma unroll
      for (int st = 0; st < KS; ++st) s = Op<T>::mfma(as_op<T>(kf[kb][st]), as_op<T>(qf[st]), s);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = kb * 16 + lg * 4 + i;
        const float v = key < n_valid ? s[i] * p.scale_log2 : -INFINITY;
        x[kb][i] = v;
        mx = fmaxf(mx, v);
      }
    }
    mx = wave_max_xor(mx, 16);
    mx = wave_max_xor(mx, 32);
    const float m_new = fmaxf(m, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m - m_use);
    m = m_new;
    float ps = 0.f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float pv = fast_exp2(x[kb][i] - m_use);
        ps += pv;
        if (lr < GT) p_lds[wave][kb * 16 + lg * 4 + i][lr] = pv;
      }
    lsum = lsum * alpha + ps;

    // rescale the P.V accumulators by each query's alpha (held by lane g)
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      const float ag = __shfl(alpha, g, 64);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[g][e] *= ag;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

#pragma unroll
    for (int jj = 0; jj < VL; ++jj) {
      const int row = jj * RPL + vrow;
      float pr[GT];
#pragma unroll
      for (int g = 0; g < GT; ++g) pr[g] = p_lds[wave][row][g];
      const u32x4 w = vf[jj];
      float vv[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vv[2 * e] = Op<T>::to_float((uint16_t)(w[e] & 0xFFFFu));
        vv[2 * e + 1] = Op<T>::to_float((uint16_t)(w[e] >> 16));
      }
#pragma unroll
      for (int g = 0; g < GT; ++g)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[g][e] = fmaf(pr[g], vv[e], acc[g][e]);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // reduce over the lanes that share a V chunk (different key rows)
#pragma unroll
  for (int msk = CPR; msk < 64; msk <<= 1)
#pragma unroll
    for (int g = 0; g < GT; ++g)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[g][e] = wave_sum_xor(acc[g][e], msk);
  lsum = wave_sum_xor(lsum, 16);
  lsum = wave_sum_xor(lsum, 32);

  if (lane < GT) {
    st_m[wave][lane] = m;
    st_l[wave][lane] = lsum;
  }
  if (vrow == 0) {
#pragma unroll
    for (int g = 0; g < GT; ++g)
#pragma unroll
      for (int e = 0; e < 8; ++e) o_lds[wave][g][vch * 8 + e] = acc[g][e];
  }
  __syncthreads();

  // merge the four waves' states and write the normalised partial
  for (int i = tid; i < G * D; i += kThreads) {
    const int g = i / D, d = i % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, st_m[w][g]);
    float den = 0.f, num = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float sc = st_m[w][g] == -INFINITY ? 0.f : fast_exp2(st_m[w][g] - M);
      den += sc * st_l[w][g];
      num += sc * o_lds[w][g][d];
    }
    const int64_t row = out_row0 + (int64_t)g * p.num_splits;
    p.part_o[row * D + d] = den > 0.f ? num / den : 0.f;
    if (d == 0) p.part_lse[row] = den > 0.f ? (M + __log2f(den)) * kLn2 : -INFINITY;
  }
}

// One wave per (sequence, head): lane s holds split s's lse.
template <int D>
__global__ __launch_bounds__(kThreads) void combine_kernel(const CombineParams p) {
  constexpr int PER = D / 64;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int pair = blockIdx.x * kWaves + wave;
  if (pair >= p.pairs) return;
  const int S = p.num_splits;
  const float l = lane < S ? p.part_lse[(int64_t)pair * S + lane] : -INFINITY;
  float M = l;
#pragma unroll
  for (int msk = 1; msk < 64; msk <<= 1) M = wave_max_xor(M, msk);
  const float w = (M == -INFINITY || l == -INFINITY) ? 0.f : fast_exp2((l - M) * kLog2e);
  float den = w;
#pragma unroll
  for (int msk = 1; msk < 64; msk <<= 1) den = wave_sum_xor(den, msk);

  float o[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) o[e] = 0.f;
  for (int s = 0; s < S; ++s) {
    const float ws = __shfl(w, s, 64);
    if (ws == 0.f) continue;                      // empty split: its O_s is never read
    const float* src = p.part_o + ((int64_t)pair * S + s) * D + lane * PER;
#pragma unroll
    for (int e = 0; e < PER; ++e) o[e] = fmaf(ws, src[e], o[e]);
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  const int64_t ob = (int64_t)pair * D + lane * PER;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const float v = o[e] * inv;
    if (p.o_dtype == kF32) static_cast<float*>(p.o)[ob + e] = v;
    else if (p.o_dtype == kF16) static_cast<uint16_t*>(p.o)[ob + e] = Op<F16>::from_float(v);
    else static_cast<uint16_t*>(p.o)[ob + e] = Op<BF16>::from_float(v);
  }
  if (p.lse && lane == 0) p.lse[pair] = den > 0.f ? M + __logf(den) : -INFINITY;
}

template <int D, typename T>
hipError_t launch_split_t(const DecodeParams& p, hipStream_t s) {
  const dim3 grid(p.num_splits, p.hkv, p.batch);
  if (p.group <= 1) hipLaunchKernelGGL((decode_split_kernel<D, T, 1>), grid, dim3(kThreads), 0, s, p);
  else if (p.group <= 2) hipLaunchKernelGGL((decode_split_kernel<D, T, 2>), grid, dim3(kThreads), 0, s, p);
  else if (p.group <= 4) hipLaunchKernelGGL((decode_split_kernel<D, T, 4>), grid, dim3(kThreads), 0, s, p);
  else if (p.group <= 8) hipLaunchKernelGGL((decode_split_kernel<D, T, 8>), grid, dim3(kThreads), 0, s, p);
  else hipLaunchKernelGGL((decode_split_kernel<D, T, 16>), grid, dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_split_d(const DecodeParams& p, int qkv_dtype, hipStream_t s) {
  return qkv_dtype == kF16 ? launch_split_t<D, F16>(p, s) : launch_split_t<D, BF16>(p, s);
}

}  // namespace

hipError_t launch_decode_split(const DecodeParams& p, int head_dim, int qkv_dtype,
                               hipStream_t stream) {
  switch (head_dim) {
    case 64: return launch_split_d<64>(p, qkv_dtype, stream);
    case 128: return launch_split_d<128>(p, qkv_dtype, stream);
    case 256: return launch_split_d<256>(p, qkv_dtype, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_combine(const CombineParams& p, int head_dim, hipStream_t stream) {
  const dim3 grid((p.pairs + kWaves - 1) / kWaves);
  switch (head_dim) {
    case 64: hipLaunchKernelGGL(combine_kernel<64>, grid, dim3(kThreads), 0, stream, p); break;
    case 128: hipLaunchKernelGGL(combine_kernel<128>, grid, dim3(kThreads), 0, stream, p); break;
    case 256: hipLaunchKernelGGL(combine_kernel<256>, grid, dim3(kThreads), 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace attn
