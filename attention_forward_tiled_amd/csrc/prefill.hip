// Tiled attention forward (prefill) for gfx950.
//
// What is computed: the online-softmax recurrence of the page "gfx942 unified
// attention, from the math up", section 3 (running max m, denominator l and
// un-normalised output o per query row, rescaled by alpha = 2^(m_old - m_new) in the
// base-2 domain, O = o / l at the end), over 64-key tiles, with the bottom-right
// causal mask and early exit of section 4 and the paged K/V gather of section 5.
//
// How it is mapped onto CDNA4:
//   * A workgroup is 4 waves and owns 128 query rows that share one KV head: for a
//     GQA group of G query heads it takes bq = 128 / G positions of every head of the
//     group, so each K/V tile read from HBM serves all G heads.
//   * Each wave owns 32 rows (two 16-row blocks). Scores are produced transposed,
//     S^T = K Q^T, with v_mfma_f32_16x16x32: K comes from LDS as the A operand and Q
//     stays in registers as the B operand for the whole kernel. The accumulator then
//     holds, per lane, one query row and 16 keys, which is exactly the B-operand
//     layout the P.V product needs, so P never leaves registers.
//   * O^T += V^T P^T with the same MFMA; the V^T operand is read from the row-major
//     V tile with ds_read_b64_tr_b16, which transposes 4x4 blocks of 16-bit values
//     on the way out of LDS. K and V are therefore stored in LDS exactly as they sit
//     in memory (row-major, 16-byte chunks XOR-swizzled by row to spread banks).
//   * K/V tiles are double-buffered in LDS: the next tile's global loads are issued
//     before the current tile's MFMAs and written to the other buffer afterwards, so
//     one barrier per tile suffices.
//   * Rows past a sequence's key length are written to LDS as zeros, so NaN or
//     garbage in unused page slots never meets a zero probability in P.V.
//   * The workgroup order is reversed over query blocks so that, under a causal
//     mask, the longest-running blocks are dispatched first.
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

// Wave-uniform byte address of a shared-memory location.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane(
      (uint32_t)(size_t)(const __attribute__((address_space(3))) void*)(p));
}

// One 16-byte-per-lane global -> LDS copy (global_load_lds_dwordx4): lane l's 16 bytes land
// at LDS byte lds + 16 * l. Issued from inline asm so that the compiler does not fence LDS
// reads of the other stage on it; completion is awaited explicitly (vmcnt) before the
// barrier that publishes the stage.
__device__ __forceinline__ void dma16(const uint16_t* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(g), "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory");
}

// Read-only device int through the constant address space, so it becomes a scalar load.
__device__ __forceinline__ int scalar_load(const int32_t* p) {
  return *(const __attribute__((address_space(4))) int32_t*)(p);
}

// 16-byte chunk swizzle: spreads the 16 rows read by one 16-lane group over 256 bytes
// of banks. Rows of 128 bytes (d = 64) pair up before the XOR so that two consecutive
// rows, which already sit in opposite bank halves, share one XOR value.
template <int D>
__device__ __forceinline__ int swz(int row) {
  if constexpr (D == 64) return (row >> 1) & 7;
  else return row & 15;
}

template <int D>
__device__ __forceinline__ int lds_off(int row, int col) {  // col in elements, multiple of 4
  return row * D + (((col >> 3) ^ swz<D>(row)) << 3) + (col & 7);
}

template <int D, typename T, bool PRECISE>
__global__ __launch_bounds__(kThreads, D == 256 ? 1 : 2) void prefill_kernel(const PrefillParams p) {
  constexpr int KS = D / 32;            // k-steps of the S^T product
  constexpr int DB = D / 16;            // 16-wide d blocks of O^T
  constexpr int CPR = D / 8;            // 16-byte chunks per row
  constexpr int RPI = 512 / D;          // rows covered by one 1 KiB wave-wide LDS load
  constexpr int NIW = kPage / RPI / kWaves;   // such loads per wave per tile (K and V each)
  constexpr int TILE = kPage * D;       // elements per K (or V) tile
  extern __shared__ __align__(16) uint16_t smem[];   // [2 stages][K, V][TILE]

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lr = lane & 15, lg = lane >> 4;
  const int qblk = gridDim.x - 1 - blockIdx.x;
  const int kvh = blockIdx.y, b = blockIdx.z;

  int L = p.seqlen_k;
  if (p.seqlens_k) L = min(max(p.seqlens_k[b], 0), p.seqlen_k);
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

  const int pmax = min(q0 + p.bq, p.seqlen_q) - 1;
  const int kv_end = p.causal ? min(L, pmax + off + 1) : L;
  const int n_tiles = kv_end > 0 ? (kv_end + kPage - 1) / kPage : 0;

  // ---- K/V tile loads straight into LDS (global_load_lds_dwordx4). One wave-wide load
  // fills 1 KiB = RPI rows; lane l lands at byte 16*l of it, so the XOR swizzle is applied
  // by choosing which 16-byte chunk of its row each lane fetches. Rows past the key length
  // (or of an invalid page) fetch a 16-byte block of zeros instead.
  const int r_in = lane / CPR, pc = lane % CPR;
  auto issue_tile = [&](int j, int stage) {
    int64_t base;
    int64_t rs;
    bool page_ok = true;
    if (p.block_table) {
      const int pg = scalar_load(p.block_table + (int64_t)b * p.max_blocks + j);
      page_ok = pg >= 0 && pg < p.num_blocks;
      base = (int64_t)(page_ok ? pg : 0) * kPage * p.hkv * D + (int64_t)kvh * D;
      rs = (int64_t)p.hkv * D;
    } else {
      base = b * p.kv_sb + kvh * p.kv_sh + (int64_t)j * kPage * p.kv_ss;
      rs = p.kv_ss;
    }
    const uint32_t ks = lds_addr(smem + stage * 2 * TILE);
    const uint32_t vs = ks + TILE * sizeof(uint16_t);
#pragma unroll
    for (int k = 0; k < NIW; ++k) {
      const int i = wave * NIW + k;
      const int r = i * RPI + r_in;
      const bool ok = page_ok && (j * kPage + r < L);
      const int64_t e = base + r * rs + ((pc ^ swz<D>(r)) << 3);
      dma16(ok ? p.k + e : kZeroChunk, ks + i * 1024);
      dma16(ok ? p.v + e : kZeroChunk, vs + i * 1024);
    }
  };

  float mref[2] = {-INFINITY, -INFINITY};   // reference max (log2 domain) of o and l
  float lsum[2] = {0.f, 0.f};
  float4v acc[DB][2];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db][0] = acc[db][1] = float4v{0, 0, 0, 0};

  if (n_tiles > 0) issue_tile(0, 0);

  for (int j = 0; j < n_tiles; ++j) {
    // tile j has landed (own loads), every wave is past tile j-1: publish and recycle
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
    if (j + 1 < n_tiles) issue_tile(j + 1, (j + 1) & 1);
    const uint16_t* ks = smem + (j & 1) * 2 * TILE;
    const uint16_t* vs = ks + TILE;

    // ---- S^T = K Q^T for 64 keys x 32 queries
    float4v s[4][2];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      s[kb][0] = s[kb][1] = float4v{0, 0, 0, 0};
#pragma unroll
      for (int st = 0; st < KS; ++st) {
        const int row = kb * 16 + lr;
        const u32x4 a = *reinterpret_cast<const u32x4*>(ks + lds_off<D>(row, st * 32 + lg * 8));
        s[kb][0] = Op<T>::mfma(as_op<T>(a), as_op<T>(qf[0][st]), s[kb][0]);
        s[kb][1] = Op<T>::mfma(as_op<T>(a), as_op<T>(qf[1][st]), s[kb][1]);
      }
    }

    // ---- online softmax (base-2 domain) with a lazily moved reference maximum: o and l
    // are kept relative to mref, which only moves (rescaling o and l by 2^(old - new)) when
    // a row's maximum exceeds it by more than kLazy; every p stays <= 2^kLazy.
    const bool need_mask = (j * kPage + kPage - 1 >= L) ||
                           (p.causal && j * kPage + kPage - 1 > q0 + off);
    float mt[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v = s[kb][qb][i];
          if (need_mask) {
            const int key = j * kPage + kb * 16 + lg * 4 + i;
            const bool vis = key < L && (!p.causal || key <= rpos[qb] + off);
            v = vis ? v : -INFINITY;
            s[kb][qb][i] = v;
          }
          mx = fmaxf(mx, v);
        }
      mx = wave_max_xor(mx, 16);
      mx = wave_max_xor(mx, 32);
      mt[qb] = mx * c;
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
      float ps = 0.f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[kb][i] = fast_exp2(__builtin_fmaf(s[kb][qb][i], c, mneg));
          ps += x[kb][i];
        }
      lsum[qb] += ps;
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
    }

    // ---- O^T += V^T P^T; V^T fragments come from the row-major tile via transpose reads
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const int row0 = s2 * 32 + 4 * lg + (lr >> 2);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int col = db * 16 + 4 * (lr & 3);
        const u32x2 lo = lds_read_tr16(vs + lds_off<D>(row0, col));
        const u32x2 hi = lds_read_tr16(vs + lds_off<D>(row0 + 16, col));
        const u32x4 a = u32x4{lo[0], lo[1], hi[0], hi[1]};
        acc[db][0] = Op<T>::mfma(as_op<T>(a), as_op<T>(pf[0][s2]), acc[db][0]);
        acc[db][1] = Op<T>::mfma(as_op<T>(a), as_op<T>(pf[1][s2]), acc[db][1]);
        if constexpr (PRECISE) {
          acc[db][0] = Op<T>::mfma(as_op<T>(a), as_op<T>(pl[0][s2]), acc[db][0]);
          acc[db][1] = Op<T>::mfma(as_op<T>(a), as_op<T>(pl[1][s2]), acc[db][1]);
        }
      }
    }
  }

  // ---- epilogue: O = o / l, lse = ln 2 * (mref + log2 l)
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    float l = wave_sum_xor(lsum[qb], 16);
    l = wave_sum_xor(l, 32);
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
