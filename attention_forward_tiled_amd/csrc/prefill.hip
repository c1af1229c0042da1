// Tiled attention forward (prefill) for gfx950.
//
// What is computed: the online-softmax recurrence of the page "gfx942 unified
// attention, from the math up", section 3 (running max m, denominator l and
// un-normalised output o per query row, O = o / l at the end), over 64-key tiles, with
// the bottom-right causal mask and early exit of section 4 and the paged K/V gather of
// section 5. Scores are handled in the base-2 domain (s * tau * log2 e, exp2).
//
// How it is mapped onto CDNA4:
//   * A workgroup is 4 waves and owns 128 query rows that share one KV head: for a
//     GQA group of G query heads it takes bq = 128 / G positions of every head of the
//     group, so each K/V tile brought into LDS serves all G heads.
//   * Each wave owns 32 rows (two 16-row blocks). Scores are produced transposed,
//     S^T = K Q^T, with v_mfma_f32_16x16x32: K comes from LDS as the A operand and Q
//     stays in registers as the B operand for the whole kernel. The accumulator then
//     holds, per lane, one query row and 16 keys, which is exactly the B-operand
//     layout the P.V product needs, so P never leaves registers.
//   * O^T += V^T P^T with the same MFMA; the V^T operand is read from the row-major
//     V tile with ds_read_b64_tr_b16, which transposes 4x4 blocks of 16-bit values
//     on the way out of LDS. K and V are therefore stored in LDS exactly as they sit
//     in memory (row-major, 16-byte chunks XOR-swizzled by row to spread banks), and
//     are copied there by global_load_lds_dwordx4 without passing through registers.
//   * Two LDS stages: tile j+1 is in flight while tile j is consumed; one barrier per
//     tile. The main loop is unrolled by two so every LDS offset is an immediate.
//   * Tiles entirely inside the visible region run a loop with no masking code; the
//     tiles that straddle the causal diagonal or the key length run a second loop that
//     masks scores and fetches rows past the key length from a block of zeros (NaN in
//     unused page slots never meets a zero probability in P.V).
//   * The reference maximum behind o and l moves lazily: only when a row's maximum
//     exceeds it by more than 2^8, so the O rescale is skipped on most tiles.
//   * Row sums of P are taken from the packed 16-bit P with v_dot2 (the same values
//     the P.V MFMA consumes).
//   * The workgroup order is reversed over query blocks so that, under a causal
//     mask, the longest-running blocks are dispatched first.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace attn {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kLazy = 8.0f;          // log2-domain slack before the reference max moves
constexpr unsigned kWaitVm0 = 0x0F70;  // s_waitcnt vmcnt(0), other counters untouched

// 16 bytes of zeros in global memory: the source of every LDS row past a key length.
__device__ __align__(16) const uint16_t kZeroChunk[8] = {0, 0, 0, 0, 0, 0, 0, 0};

// Byte address of a shared-memory location.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(size_t)(const __attribute__((address_space(3))) void*)(p);
}

// global_load_lds_dwordx4 with a per-lane 64-bit address: lane l's 16 bytes land at LDS
// byte lds + 16 * l. Issued from inline asm so that the compiler does not fence LDS reads
// of the other stage on it; completion is awaited explicitly (vmcnt) before the barrier
// that publishes the stage.
__device__ __forceinline__ void dma16_v(const uint16_t* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(g), "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory");
}

// Same copy with a wave-uniform base in SGPRs and a per-lane 32-bit byte offset.
__device__ __forceinline__ void dma16_s(const uint16_t* base, uint32_t voff, uint32_t lds) {
  // readfirstlane returns a signed int: widen through uint32_t so the low word is not
  // sign-extended into the high one.
  const uint64_t b = (uint64_t)base;
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint64_t bs = ((uint64_t)hi << 32) | (uint64_t)lo;
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(voff), "s"((const uint16_t*)bs), "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory");
}

// Read-only device int through the constant address space, so it becomes a scalar load.
__device__ __forceinline__ int scalar_load(const int32_t* p) {
  return *(const __attribute__((address_space(4))) int32_t*)(p);
}

// 16-byte chunk swizzle: spreads the 16 rows read by one 16-lane group over 256 bytes
// of banks. Rows of 128 bytes (d = 64) pair up before the XOR so that two consecutive
// rows, which already sit in opposite bank halves, share one XOR value. Only row % 16
// (row % 32 for d = 64, through row >> 1) matters, so rows 16 apart share a pattern.
template <int D>
__device__ __forceinline__ int swz(int row) {
  if constexpr (D == 64) return (row >> 1) & 7;
  else return row & 15;
}

template <int D, typename T, bool PRECISE>
__global__ __launch_bounds__(kThreads, D == 256 ? 1 : 2) void prefill_kernel(const PrefillParams p) {
  constexpr int KS = D / 32;            // k-steps of the S^T product
  constexpr int DB = D / 16;            // 16-wide d blocks of O^T
  constexpr int CPR = D / 8;            // 16-byte chunks per row
  constexpr int RPI = 512 / D;          // rows covered by one 1 KiB wave-wide LDS copy
  constexpr int NIW = kPage / RPI / kWaves;   // such copies per wave per tile (K and V each)
  constexpr int TILE = kPage * D;       // elements per K (or V) tile
  constexpr int ROWB = D * 2;           // bytes per LDS row
  extern __shared__ __align__(16) uint16_t smem[];   // [2 stages][K, V][TILE]

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lr = lane & 15, lg = lane >> 4;
  const int qblk = gridDim.x - 1 - blockIdx.x;
  const int kvh = blockIdx.y, b = blockIdx.z;

  int L = p.seqlen_k;
  if (p.seqlens_k) L = min(max(scalar_load(p.seqlens_k + b), 0), p.seqlen_k);
  const int q0 = qblk * p.bq;
  const int off = L - p.seqlen_q;       // bottom-right alignment of the causal mask
  const float c = p.scale_log2;

  // ---- this lane's two query rows (one per 16-row block) and their Q fragments
  int rpos[2], rh[2];
  bool rok[2];
  u32x4 qf[2][KS];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int r = wave * 32 + qb * 16 + lr;
    const int hig = r / p.bq;
    rpos[qb] = q0 + (r - hig * p.bq);
    rh[qb] = kvh * p.group + hig;
    rok[qb] = hig < p.group && rpos[qb] < p.seqlen_q;
    const uint16_t* qp = p.q + b * p.q_sb + (int64_t)rh[qb] * p.q_sh + (int64_t)rpos[qb] * p.q_ss;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qf[qb][s] = rok[qb] ? ldg16(qp + s * 32 + lg * 8) : u32x4{0, 0, 0, 0};
  }

  // ---- tile range: [0, n_full) need no masking, [n_full, n_tiles) straddle a boundary
  const int pmax = min(q0 + p.bq, p.seqlen_q) - 1;
  const int kv_end = p.causal ? min(L, pmax + off + 1) : L;
  const int n_tiles = kv_end > 0 ? (kv_end + kPage - 1) / kPage : 0;
  int n_full = L / kPage;
  if (p.causal) n_full = min(n_full, max(q0 + off + 1, 0) / kPage);
  n_full = min(n_full, n_tiles);

  // ---- per-lane constants of the K/V copies (byte offsets inside a tile's rows)
  const bool paged = p.block_table != nullptr;
  const int64_t rs = paged ? (int64_t)p.hkv * D : p.kv_ss;   // elements between key rows
  const int r_in = lane / CPR, pc = lane % CPR;
  uint32_t dma_off[NIW];
#pragma unroll
  for (int k = 0; k < NIW; ++k) {
    const int r = (wave * NIW + k) * RPI + r_in;
    dma_off[k] = (uint32_t)((r * rs + ((pc ^ swz<D>(r)) << 3)) * 2);
  }
  const uint32_t smem_base = lds_addr(smem);

  // Copy tile j into LDS stage `stage`. Rows past the key length, and every row of a page
  // whose id is out of range, are fetched from the zero block instead.
  auto issue_tile = [&](int j, int stage) {
    int64_t base;
    bool page_ok = true;
    if (paged) {
      const int pg = scalar_load(p.block_table + (int64_t)b * p.max_blocks + j);
      page_ok = pg >= 0 && pg < p.num_blocks;
      base = (int64_t)(page_ok ? pg : 0) * kPage * p.hkv * D + (int64_t)kvh * D;
    } else {
      base = b * p.kv_sb + kvh * p.kv_sh + (int64_t)j * kPage * p.kv_ss;
    }
    const uint32_t ks = smem_base + stage * 2 * TILE * 2;
    const uint32_t vs = ks + TILE * 2;
    if (page_ok && (j + 1) * kPage <= L) {
#pragma unroll
      for (int k = 0; k < NIW; ++k) {
        const int i = wave * NIW + k;
        dma16_s(p.k + base, dma_off[k], ks + i * 1024);
        dma16_s(p.v + base, dma_off[k], vs + i * 1024);
      }
    } else {
#pragma unroll
      for (int k = 0; k < NIW; ++k) {
        const int i = wave * NIW + k;
        const bool ok = page_ok && (j * kPage + (i * RPI + r_in) < L);
        dma16_v(ok ? p.k + base + dma_off[k] / 2 : kZeroChunk, ks + i * 1024);
        dma16_v(ok ? p.v + base + dma_off[k] / 2 : kZeroChunk, vs + i * 1024);
      }
    }
  };

  // ---- per-lane LDS read offsets (bytes inside a stage's K or V tile)
  // K A-operand for S^T: row kb*16 + lr, chunk 4*st + lg (kb enters as an immediate).
  uint32_t koff[KS];
#pragma unroll
  for (int st = 0; st < KS; ++st) koff[st] = lr * ROWB + (((st * 4 + lg) ^ swz<D>(lr)) << 4);
  // V^T A-operand via transpose reads: lane (lg, lr) addresses row 4*lg + lr/4 (+16, +32)
  // at column 16*db + 4*(lr % 4).
  const int vrow = 4 * lg + (lr >> 2);
  uint32_t voff[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    const int chunk = 2 * db + ((lr & 3) >> 1);
    voff[db] = vrow * ROWB + ((chunk ^ swz<D>(vrow)) << 4) + 8 * (lr & 1);
  }

  float mref[2] = {-INFINITY, -INFINITY};   // reference max (log2 domain) of o and l
  float lsum[2] = {0.f, 0.f};               // this lane's share of l
  float4v acc[DB][2];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db][0] = acc[db][1] = float4v{0, 0, 0, 0};

  // One tile: S^T = K Q^T, online softmax, O^T += V^T P^T.
  auto step = [&](int j, auto stage_c, auto mask_c) {
    constexpr int STAGE = decltype(stage_c)::value;
    constexpr bool MASK = decltype(mask_c)::value;
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
    if (j + 1 < n_tiles) issue_tile(j + 1, STAGE ^ 1);
    const char* ks = reinterpret_cast<const char*>(smem) + STAGE * 2 * TILE * 2;
    const char* vs = ks + TILE * 2;

    float4v s[4][2];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      s[kb][0] = s[kb][1] = float4v{0, 0, 0, 0};
#pragma unroll
      for (int st = 0; st < KS; ++st) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(ks + koff[st] + kb * 16 * ROWB);
        s[kb][0] = Op<T>::mfma(as_op<T>(a), as_op<T>(qf[0][st]), s[kb][0]);
        s[kb][1] = Op<T>::mfma(as_op<T>(a), as_op<T>(qf[1][st]), s[kb][1]);
      }
    }

    float mt[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      if constexpr (MASK) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = j * kPage + kb * 16 + lg * 4 + i;
            const bool vis = key < L && (!p.causal || key <= rpos[qb] + off);
            s[kb][qb][i] = vis ? s[kb][qb][i] : -INFINITY;
          }
      }
      float mx = s[0][qb][0];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (kb | i) mx = fmaxf(mx, s[kb][qb][i]);
      mt[qb] = rows4_max(mx) * c;
    }
    const bool up0 = mt[0] > mref[0] + kLazy, up1 = mt[1] > mref[1] + kLazy;
    if (__builtin_amdgcn_ballot_w64(up0 || up1) != 0) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const bool up = qb ? up1 : up0;
        const float nref = up ? mt[qb] : mref[qb];
        const float alpha = up ? fast_exp2(mref[qb] - nref) : 1.f;
        mref[qb] = nref;
        lsum[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[db][qb] *= alpha;
      }
    }

    u32x4 pf[2][2];
    u32x4 pl[2][2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const float mneg = mref[qb] == -INFINITY ? 0.f : -mref[qb];
      float x[4][4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) x[kb][i] = fast_exp2(__builtin_fmaf(s[kb][qb][i], c, mneg));
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const float* a0 = x[2 * s2];
        const float* a1 = x[2 * s2 + 1];
        pf[qb][s2] = u32x4{pack2<T>(a0[0], a0[1]), pack2<T>(a0[2], a0[3]),
                           pack2<T>(a1[0], a1[1]), pack2<T>(a1[2], a1[3])};
        if constexpr (PRECISE) {
          float r0[4], r1[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            r0[i] = a0[i] - Op<T>::to_float(Op<T>::from_float(a0[i]));
            r1[i] = a1[i] - Op<T>::to_float(Op<T>::from_float(a1[i]));
          }
          pl[qb][s2] = u32x4{pack2<T>(r0[0], r0[1]), pack2<T>(r0[2], r0[3]),
                             pack2<T>(r1[0], r1[1]), pack2<T>(r1[2], r1[3])};
        }
      }
      if constexpr (PRECISE) {
        float ps = 0.f;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) ps += x[kb][i];
        lsum[qb] += ps;
      } else {
        float ps0 = lsum[qb], ps1 = 0.f;
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          ps0 = Op<T>::sum2(pf[qb][s2][0], ps0);
          ps1 = Op<T>::sum2(pf[qb][s2][1], ps1);
          ps0 = Op<T>::sum2(pf[qb][s2][2], ps0);
          ps1 = Op<T>::sum2(pf[qb][s2][3], ps1);
        }
        lsum[qb] = ps0 + ps1;
      }
    }

#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const u32x2 lo = lds_read_tr16(reinterpret_cast<const uint16_t*>(vs + voff[db] + s2 * 32 * ROWB));
        const u32x2 hi = lds_read_tr16(reinterpret_cast<const uint16_t*>(vs + voff[db] + (s2 * 32 + 16) * ROWB));
        const u32x4 a = u32x4{lo[0], lo[1], hi[0], hi[1]};
        acc[db][0] = Op<T>::mfma(as_op<T>(a), as_op<T>(pf[0][s2]), acc[db][0]);
        acc[db][1] = Op<T>::mfma(as_op<T>(a), as_op<T>(pf[1][s2]), acc[db][1]);
        if constexpr (PRECISE) {
          acc[db][0] = Op<T>::mfma(as_op<T>(a), as_op<T>(pl[0][s2]), acc[db][0]);
          acc[db][1] = Op<T>::mfma(as_op<T>(a), as_op<T>(pl[1][s2]), acc[db][1]);
        }
      }
    }
  };

  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using Full = std::integral_constant<bool, false>;
  using Masked = std::integral_constant<bool, true>;

  if (n_tiles > 0) issue_tile(0, 0);
  int j = 0;
  for (; j + 1 < n_full; j += 2) {
    step(j, S0{}, Full{});
    step(j + 1, S1{}, Full{});
  }
  if (j < n_full) {
    step(j, S0{}, Full{});
    ++j;
  }
  for (; j < n_tiles; ++j) {
    if (j & 1) step(j, S1{}, Masked{});
    else step(j, S0{}, Masked{});
  }

  // ---- epilogue: O = o / l, lse = ln 2 * (mref + log2 l)
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float l = rows4_sum(lsum[qb]);
    if (!rok[qb]) continue;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const int64_t ob = b * p.o_sb + (int64_t)rh[qb] * p.o_sh + (int64_t)rpos[qb] * p.o_ss;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int d0 = db * 16 + lg * 4;
      const float4v v = acc[db][qb] * inv;
      if (p.o_dtype == kF32) {
        *reinterpret_cast<float4v*>(static_cast<float*>(p.o) + ob + d0) = v;
      } else if (p.o_dtype == kF16) {
        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(p.o) + ob + d0) =
            u32x2{pack2<F16>(v[0], v[1]), pack2<F16>(v[2], v[3])};
      } else {
        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(p.o) + ob + d0) =
            u32x2{pack2<BF16>(v[0], v[1]), pack2<BF16>(v[2], v[3])};
      }
    }
    if (p.lse && lg == 0)
      p.lse[((int64_t)b * p.hq + rh[qb]) * p.seqlen_q + rpos[qb]] =
          l > 0.f ? (mref[qb] + __log2f(l)) * kLn2 : -INFINITY;
  }
}

template <int D, typename T, bool PRECISE>
hipError_t launch_one(const PrefillParams& p, hipStream_t stream) {
  const size_t lds = 2 * 2 * kPage * D * sizeof(uint16_t);
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill_kernel<D, T, PRECISE>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const dim3 grid((p.seqlen_q + p.bq - 1) / p.bq, p.hkv, p.batch);
  hipLaunchKernelGGL((prefill_kernel<D, T, PRECISE>), grid, dim3(kThreads), lds, stream, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const PrefillParams& p, int qkv_dtype, bool precise, hipStream_t s) {
  if (qkv_dtype == kF16)
    return precise ? launch_one<D, F16, true>(p, s) : launch_one<D, F16, false>(p, s);
  return precise ? launch_one<D, BF16, true>(p, s) : launch_one<D, BF16, false>(p, s);
}

}  // namespace

hipError_t launch_prefill(const PrefillParams& p, int head_dim, int qkv_dtype, bool precise,
                          hipStream_t stream) {
  switch (head_dim) {
    case 64: return launch_d<64>(p, qkv_dtype, precise, stream);
    case 128: return launch_d<128>(p, qkv_dtype, precise, stream);
    case 256: return launch_d<256>(p, qkv_dtype, precise, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace attn
