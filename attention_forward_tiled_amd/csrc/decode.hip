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
// How it is mapped onto CDNA4. The split kernel streams every K/V byte once from HBM
// and does little arithmetic per byte, so its design is about keeping enough bytes in
// flight, not about flops:
//   * One workgroup (4 waves) per (KV head, sequence, partition), launched partition-
//     major so that the first partitions of every sequence, which are always full,
//     are dispatched first and the partial tail partitions fill the end of the grid.
//     The G query heads that share the KV head are processed together, so every K/V
//     byte is read once.
//   * Pages stream through a ring of LDS stages (K tile and V tile of one 64-key page
//     per stage) filled by global_load_lds_dwordx4, which needs no registers for the
//     data in flight; the ring is several pages deep, and page i + NST - 1 is started
//     as soon as page i is published, so up to NST - 1 pages are in flight while page
//     i is consumed.
//   * All four waves work on the same page, 16 keys each: S^T = K Q^T with
//     v_mfma_f32_16x16x32 (K rows from LDS as the A operand, the group's query heads
//     padded to 16 columns as the B operand). The accumulator layout is the B-operand
//     layout of v_mfma_f32_16x16x16, so O^T += V^T P^T follows with P in registers and
//     V^T read from the row-major V tile by ds_read_b64_tr_b16. Each wave keeps its own
//     (m, l, o) per query head; the four are merged through LDS at the end.
//   * Rows past the partition end and rows of pages whose id is out of range are
//     copied from a block of zeros and their scores are masked, so NaN in unused page
//     slots never reaches the output.
#include "common.hpp"
#include "kernels.hpp"

namespace attn {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

// 16-byte chunk swizzle of the decode's LDS tiles, chunk' = chunk ^ dswz(row). It keeps
// two read patterns free of bank conflicts: the K reads (16 consecutive rows at one chunk
// per 16 lanes) and the V transpose reads (8 consecutive rows times two adjacent chunks
// per 32 lanes). For rows of 256 bytes or more, row r maps to 2 * (r mod 8) + (r / 8 mod
// 2): a permutation of 0..15 whose upper three bits differ inside each run of 8 rows. For
// d = 64 (two 128-byte rows per 256 bytes) the same idea is applied to row / 2 mod 8.
template <int D>
__device__ __forceinline__ int dswz(int row) {
  if constexpr (D == 64) {
    const int k = (row >> 1) & 7;
    return ((k & 3) << 1) | (k >> 2);
  } else {
    const int r = row & 15;
    return ((r & 7) << 1) | (r >> 3);
  }
}

// Wait until at most `ahead` pages of copies (PER wave-instructions each) are still in
// flight for this wave; `ahead` is at most N. The count has to be an immediate.
template <int PER, int N>
__device__ __forceinline__ void wait_pages(int ahead) {
  if constexpr (N <= 0) {
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
  } else {
    if (ahead >= N) __builtin_amdgcn_s_waitcnt(wait_vm(N * PER));
    else wait_pages<PER, N - 1>(ahead);
  }
}

// Ring depth: 128 KiB of K/V stages per workgroup.
template <int D> constexpr int kDecodeStages = 512 / D;

template <int D, typename T, int NST>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(const DecodeParams p) {
  constexpr int KS = D / 32;                 // k-steps of S^T
  constexpr int DB = D / 16;                 // 16-wide d blocks of O^T
  constexpr int CPR = D / 8;                 // 16-byte chunks per key row
  constexpr int RPI = 512 / D;               // rows per 1 KiB wave-wide copy
  constexpr int NIW = kPage / RPI / kWaves;  // such copies per wave per tile (K and V each)
  constexpr int ROWB = D * 2;                // bytes per LDS row
  constexpr int TILE_B = kPage * ROWB;       // bytes per K (or V) tile
  constexpr int OSTR = D + 4;                // floats per row of the merge buffer (padded)
  static_assert(NST >= 2 && (NST - 2) * 2 * NIW < 64, "ring depth");
  static_assert(kWaves * 16 * OSTR * 4 + 2 * kWaves * 16 * 4 <= NST * 2 * TILE_B, "merge buffer");
  __shared__ __align__(16) char ring[NST * 2 * TILE_B];   // [stage][K, V][64 rows][D]

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lr = lane & 15, lg = lane >> 4;
  const int kvh = blockIdx.x, b = blockIdx.y, split = blockIdx.z;
  const int G = p.group;

  const int L = min(max(scalar_load(p.seqlens_k + b), 0), p.max_seqlen_k);
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

  // Q fragments (B operand of S^T): lane lr holds query head lr of the group (zero if
  // lr >= G). They are waited for here, before any copy is started, so that the wait
  // the compiler places before their first use does not also drain the copies.
  u32x4 qf[KS];
  {
    const bool ok = lr < G;
    const uint16_t* qp = p.q + ((int64_t)b * p.hq + (int64_t)kvh * G + (ok ? lr : 0)) * D;
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = ok ? ldg16(qp + s * 32 + lg * 8) : u32x4{0, 0, 0, 0};
  }
  __builtin_amdgcn_s_waitcnt(kWaitVm0);

  const int first_page = start / kPage;            // start is a multiple of the page size
  const int n_pages = (end - start + kPage - 1) / kPage;
  const int64_t rs = (int64_t)p.hkv * D;           // elements between key rows of a page
  const int32_t* table = p.block_table + (int64_t)b * p.max_blocks + first_page;

  // per-lane byte offsets of the copies inside a page (row-major, swizzled chunks)
  const int r_in = lane / CPR, pc = lane % CPR;
  uint32_t dma_off[NIW];
#pragma unroll
  for (int k = 0; k < NIW; ++k) {
    const int row = (wave * NIW + k) * RPI + r_in;
    dma_off[k] = (uint32_t)((row * rs + ((pc ^ dswz<D>(row)) << 3)) * 2);
  }
  const uint32_t ring_base = lds_addr(ring);
  uint32_t page_ok_bits = 0;   // bit (k mod 32): page k of this partition has a valid id

  // Start the copies of page k into stage k % NST.
  auto issue = [&](int k) __attribute__((always_inline)) {
    const int pg = scalar_load(table + k);
    const bool page_ok = pg >= 0 && pg < p.num_blocks;
    page_ok_bits = (page_ok_bits & ~(1u << (k & 31))) | ((uint32_t)page_ok << (k & 31));
    const int64_t base = (int64_t)(page_ok ? pg : 0) * kPage * rs + (int64_t)kvh * D;
    const int key0 = start + k * kPage;
    const uint32_t ks = ring_base + (k % NST) * 2 * TILE_B;
    const uint32_t vs = ks + TILE_B;
    if (page_ok && key0 + kPage <= end) {
#pragma unroll
      for (int i = 0; i < NIW; ++i) dma16_s(p.k + base, dma_off[i], ks + (wave * NIW + i) * 1024);
#pragma unroll
      for (int i = 0; i < NIW; ++i) dma16_s(p.v + base, dma_off[i], vs + (wave * NIW + i) * 1024);
    } else {
#pragma unroll
      for (int i = 0; i < NIW; ++i) {
        const bool ok = page_ok && key0 + (wave * NIW + i) * RPI + r_in < end;
        dma16_v(ok ? p.k + base + dma_off[i] / 2 : kZeroChunk, ks + (wave * NIW + i) * 1024);
      }
#pragma unroll
      for (int i = 0; i < NIW; ++i) {
        const bool ok = page_ok && key0 + (wave * NIW + i) * RPI + r_in < end;
        dma16_v(ok ? p.v + base + dma_off[i] / 2 : kZeroChunk, vs + (wave * NIW + i) * 1024);
      }
    }
  };

  // per-lane LDS read offsets inside a stage's K / V tile
  uint32_t koff[KS];
  {
    const int row = 16 * wave + lr;
#pragma unroll
    for (int s = 0; s < KS; ++s) koff[s] = row * ROWB + (((4 * s + lg) ^ dswz<D>(row)) << 4);
  }
  uint32_t voff[DB];
  {
    const int row = 16 * wave + 4 * lg + (lr >> 2);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int chunk = 2 * db + ((lr & 3) >> 1);
      voff[db] = row * ROWB + ((chunk ^ dswz<D>(row)) << 4) + 8 * (lr & 1);
    }
  }

  // running state of query head lr over this wave's keys (log2 domain)
  float m = -INFINITY, lsum = 0.f;
  float4v acc[DB];   // O^T: lane holds d = 16*db + 4*lg + i of query head lr
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = float4v{0.f, 0.f, 0.f, 0.f};

  for (int k = 0; k < min(NST - 1, n_pages); ++k) issue(k);

  for (int i = 0; i < n_pages; ++i) {
    wait_pages<2 * NIW, NST - 2>(min(NST - 2, n_pages - 1 - i));
    __syncthreads();   // page i visible to every wave; stage (i - 1) % NST free again
    if (i + NST - 1 < n_pages) issue(i + NST - 1);

    const char* kt = ring + (i % NST) * 2 * TILE_B;
    const char* vt = kt + TILE_B;
    float4v s = {0.f, 0.f, 0.f, 0.f};   // S^T: keys 16*wave + 4*lg + j, query head lr
#pragma unroll
    for (int st = 0; st < KS; ++st)
      s = Op<T>::mfma(as_op<T>(*reinterpret_cast<const u32x4*>(kt + koff[st])), as_op<T>(qf[st]), s);

    const bool page_ok = (page_ok_bits >> (i & 31)) & 1u;
    const int key = start + i * kPage + 16 * wave + 4 * lg;
    float x[4];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[j] = page_ok && key + j < end ? s[j] * p.scale_log2 : -INFINITY;
      mx = fmaxf(mx, x[j]);
    }
    mx = rows4_max(mx);
    const float m_new = fmaxf(m, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m - m_use);
    m = m_new;
    float pr[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) pr[j] = fast_exp2(x[j] - m_use);
    lsum = lsum * alpha + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
    const u32x2 pb = u32x2{pack2<T>(pr[0], pr[1]), pack2<T>(pr[2], pr[3])};
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const u32x2 a = lds_read_tr16(reinterpret_cast<const uint16_t*>(vt + voff[db]));
      acc[db] = Op<T>::mfma16k(a, pb, acc[db] * alpha);
    }
  }

  // ---- merge the four waves' states through LDS and write the normalised partial
  lsum = rows4_sum(lsum);
  __syncthreads();   // every copy has landed (the last wait drained them) and been consumed
  float* o_lds = reinterpret_cast<float*>(ring);               // [wave][16][OSTR]
  float* st_m = o_lds + kWaves * 16 * OSTR;                   // [wave][16]
  float* st_l = st_m + kWaves * 16;                           // [wave][16]
  if (lg == 0) {
    st_m[wave * 16 + lr] = m;
    st_l[wave * 16 + lr] = lsum;
  }
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j) o_lds[(wave * 16 + lr) * OSTR + 16 * db + 4 * lg + j] = acc[db][j];
  __syncthreads();

  for (int idx = tid; idx < G * D; idx += kThreads) {
    const int g = idx / D, d = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, st_m[w * 16 + g]);
    float den = 0.f, num = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = st_m[w * 16 + g];
      const float sc = mw == -INFINITY ? 0.f : fast_exp2(mw - M);
      den += sc * st_l[w * 16 + g];
      num += sc * o_lds[(w * 16 + g) * OSTR + d];
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
  // partition-major order: blockIdx.z is the partition
  const dim3 grid(p.hkv, p.batch, p.num_splits);
  hipLaunchKernelGGL((decode_split_kernel<D, T, kDecodeStages<D>>), grid, dim3(kThreads), 0, s, p);
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
