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
//     data in flight; the ring is two to four pages deep, and page i + NST - 1 is started
//     as soon as page i is published, so up to NST - 1 pages are in flight while page
//     i is consumed. The K/V copies are non-temporal: every page is read once, and
//     marking the stream so keeps it from displacing reusable cache lines (12% faster).
//     The persistent variant (decode_stream_kernel, below) is the one used for
//     num_splits >= 2. At d = 64 it consumes two pages of a partition per barrier (one
//     128-key tile), since a page there carries half the bytes for the same chain of
//     dependent steps.
//   * All four waves work on the same page, 16 keys each: S^T = K Q^T with
//     v_mfma_f32_16x16x32 (K rows from LDS as the A operand, the group's query heads
//     padded to 16 columns as the B operand). The accumulator layout is the B-operand
//     layout of v_mfma_f32_16x16x16, so O^T += V^T P^T follows with P in registers and
//     V^T read from the row-major V tile by ds_read_b64_tr_b16. Each wave keeps its own
//     (m, l, o) per query head; the four are merged through LDS at the end. The reference
//     maximum m moves only when a score exceeds it by more than 2^8, so most pages skip
//     the cross-lane maximum and the rescale. The denominator l sums P as rounded to the
//     16-bit type for the P.V product (v_dot2 on the packed values), as the prefill does,
//     so each partial output is a weighted mean of V rows whose weights sum to one.
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

// Log2-domain slack before a running reference maximum moves.
constexpr float kLazy = 8.0f;

// Reference-maximum update of one online-softmax step. m is the row's reference (its
// denominator and output accumulator are relative to it) and mx this lane's maximum over
// its new scores. The reference moves to the row maximum only when some score of the wave
// exceeds m + kLazy; otherwise the cross-lane maximum and the rescale are skipped
// (alpha = 1) and the new exponentials stay below 2^kLazy. The recurrence holds for any
// reference, so only rounding changes. Returns the value to exponentiate against.
__device__ __forceinline__ float move_ref(float& m, float mx, float& alpha) {
  if (__builtin_amdgcn_ballot_w64(mx > m + kLazy) != 0) {   // wave-uniform branch
    const float m_new = fmaxf(m, rows4_max(mx));
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    alpha = fast_exp2(m - m_use);
    m = m_new;
    return m_use;
  }
  alpha = 1.f;
  return m == -INFINITY ? 0.f : m;
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
  if constexpr (kPoisonLds) poison_lds<sizeof(ring)>(ring);

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

  const int first_page = start / kPage;            // start is a multiple of the page size
  const int n_pages = (end - start + kPage - 1) / kPage;
  const int64_t rs = (int64_t)p.hkv * D;           // elements between key rows of a page
  const int32_t* table = p.block_table + (int64_t)b * p.max_blocks + first_page;

  // Page ids are read with scalar loads ahead of their use: the first NST - 1 here, all
  // in flight together with the Q loads, and later ones one page ahead of the copy.
  int pid[NST - 1];
#pragma unroll
  for (int k = 0; k < NST - 1; ++k) pid[k] = k < n_pages ? scalar_load(table + k) : 0;
  int pid_next = NST - 1 < n_pages ? scalar_load(table + NST - 1) : 0;

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

  // Start the copies of page k (physical page pg) into stage k % NST.
  auto issue = [&](int k, int pg) __attribute__((always_inline)) {
    const bool page_ok = pg >= 0 && pg < p.num_blocks;
    page_ok_bits = (page_ok_bits & ~(1u << (k & 31))) | ((uint32_t)page_ok << (k & 31));
    const int64_t base = (int64_t)(page_ok ? pg : 0) * kPage * rs + (int64_t)kvh * D;
    const int key0 = start + k * kPage;
    const uint32_t ks = ring_base + (k % NST) * 2 * TILE_B;
    const uint32_t vs = ks + TILE_B;
    if (page_ok && key0 + kPage <= end) {
#pragma unroll
      for (int i = 0; i < NIW; ++i) dma16_s<true>(p.k + base, dma_off[i], ks + (wave * NIW + i) * 1024);
#pragma unroll
      for (int i = 0; i < NIW; ++i) dma16_s<true>(p.v + base, dma_off[i], vs + (wave * NIW + i) * 1024);
    } else {
#pragma unroll
      for (int i = 0; i < NIW; ++i) {
        const bool ok = page_ok && key0 + (wave * NIW + i) * RPI + r_in < end;
        dma16_v<true>(ok ? p.k + base + dma_off[i] / 2 : kZeroChunk, ks + (wave * NIW + i) * 1024);
      }
#pragma unroll
      for (int i = 0; i < NIW; ++i) {
        const bool ok = page_ok && key0 + (wave * NIW + i) * RPI + r_in < end;
        dma16_v<true>(ok ? p.v + base + dma_off[i] / 2 : kZeroChunk, vs + (wave * NIW + i) * 1024);
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

#pragma unroll
  for (int k = 0; k < NST - 1; ++k)
    if (k < n_pages) issue(k, pid[k]);

  for (int i = 0; i < n_pages; ++i) {
    wait_pages<2 * NIW, NST - 2>(min(NST - 2, n_pages - 1 - i));
    __syncthreads();   // page i visible to every wave; stage (i - 1) % NST free again
    if (i + NST - 1 < n_pages) {
      const int pg = pid_next;
      if (i + NST < n_pages) pid_next = scalar_load(table + i + NST);
      issue(i + NST - 1, pg);
    }

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
    float alpha;
    const float m_use = move_ref(m, mx, alpha);
    float pr[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) pr[j] = fast_exp2(x[j] - m_use);
    const u32x2 pb = u32x2{pack2<T>(pr[0], pr[1]), pack2<T>(pr[2], pr[3])};
    lsum = Op<T>::sum2(pb[1], Op<T>::sum2(pb[0], lsum * alpha));
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

// Number of 64-key pages of sequence b (its key length clamped to [0, max_seqlen_k]).
__device__ __forceinline__ int seq_pages(const DecodeParams& p, int b) {
  const int L = min(max(scalar_load(p.seqlens_k + b), 0), p.max_seqlen_k);
  return (L + kPage - 1) / kPage;
}

// Plan of the balanced decode (one workgroup of 1024 threads). The work of one KV head
// is the concatenation of the sequences' pages ("runs", sequence-major): unit u is a
// page of a run. The units are cut into `nwk` equal ranges of `chunk` units, one per
// workgroup of the stream kernel; a run cut by range boundaries becomes several
// partitions. chunk >= ceil(max pages per run / (num_splits - 1)) keeps the number of
// partitions of any run <= num_splits. Writes prefix[b] (first unit of run b, and the
// total at prefix[B]), start[j] (the run holding unit j * chunk) and plan = {total,
// chunk, nwk}.
__global__ __launch_bounds__(1024) void decode_plan_kernel(const DecodeParams p) {
  __shared__ int part[1024];
  if constexpr (kPoisonLds) poison_lds<sizeof(part)>(part);
  const int t = threadIdx.x;
  const int per = (p.batch + 1023) / 1024;
  const int b0 = min(t * per, p.batch), b1 = min(b0 + per, p.batch);
  int sum = 0;
  for (int b = b0; b < b1; ++b) sum += seq_pages(p, b);
  part[t] = sum;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {   // inclusive scan of the per-thread sums
    const int v = t >= off ? part[t - off] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  const int total = part[1023];
  int chunk = max((total + p.nwk - 1) / p.nwk, 1);
  const int rmax = (p.max_seqlen_k + kPage - 1) / kPage;
  if (p.num_splits > 1) chunk = max(chunk, (rmax + p.num_splits - 2) / (p.num_splits - 1));
  int u = part[t] - sum;
  for (int b = b0; b < b1; ++b) {
    const int r = seq_pages(p, b);
    p.prefix[b] = u;
    for (int64_t j = (u + (int64_t)chunk - 1) / chunk; j * chunk < (int64_t)u + r; ++j) p.start[j] = b;
    u += r;
  }
  if (t == 1023) {
    p.prefix[p.batch] = total;
    p.plan[0] = total;
    p.plan[1] = chunk;
    p.plan[2] = total > 0 ? (total + chunk - 1) / chunk : 0;
  }
}

// Ring depth of the stream kernel, in stages of (K tile, V tile, Q block): at d = 64
// (two pages consumed per barrier) four stages, 80 KiB, and at d = 128 two, 72 KiB, so
// that two workgroups share a CU: a second wave per SIMD hides part of the per-page chain
// of dependent steps (+2% each against one workgroup with all the LDS, eight and four
// stages). At d = 256 two stages of 72 KiB, one workgroup per CU.
template <int D> constexpr int kStreamStages = D == 64 ? 4 : 2;

// Balanced (persistent) split kernel. Workgroup w serves KV head w % Hkv and unit range
// j = w / Hkv of the plan; the workgroups of the Hkv heads with the same j walk the
// same pages at about the same time. The pages of the range stream through the ring
// without a break at partition boundaries; each page's stage also receives the G
// query rows of its run (16-row block, rows >= G zero), so that no register load is
// needed when the run changes. At the end of a partition the four waves' states are
// merged through the stage of its last page and the partial is written to slot k of
// its run, k = (first unit / chunk) - (run start / chunk); the workgroup that ends a run
// marks its unused slots with lse = -inf.
template <int D, typename T, int NST>
__global__ __launch_bounds__(kThreads) void decode_stream_kernel(const DecodeParams p) {
  constexpr int KS = D / 32;                 // k-steps of S^T
  constexpr int DB = D / 16;                 // 16-wide d blocks of O^T
  constexpr int CPR = D / 8;                 // 16-byte chunks per key row
  constexpr int RPI = 512 / D;               // rows per 1 KiB wave-wide copy
  constexpr int NIW = kPage / RPI / kWaves;  // such copies per wave per K (or V) tile
  constexpr int QIW = D >= 128 ? D / 128 : 1;   // copies per wave for the Q block
  constexpr int PER = 2 * NIW + QIW;         // copies per wave per page
  constexpr int ROWB = D * 2;                // bytes per LDS row
  constexpr int TILE_B = kPage * ROWB;       // bytes per K (or V) tile
  constexpr int STAGE_B = 2 * TILE_B + QIW * kWaves * 1024;
  constexpr bool kPairs = D == 64;           // two pages consumed per barrier
  static_assert(NST >= 2 && (NST - 2) * PER < 64, "ring depth");
  static_assert(3 * DB * 1024 + 2 * 3 * 64 * 4 <= STAGE_B, "merge buffer");
  static_assert(QIW * kWaves * 1024 >= 16 * ROWB, "Q block");
  __shared__ __align__(16) char ring[NST * STAGE_B];   // [stage][K tile, V tile, Q block]
  if constexpr (kPoisonLds) poison_lds<sizeof(ring)>(ring);

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lr = lane & 15, lg = lane >> 4;
  const int kvh = blockIdx.x % p.hkv, jr = blockIdx.x / p.hkv;
  const int G = p.group, S = p.num_splits;

  const int total = scalar_load(p.plan), chunk = scalar_load(p.plan + 1);
  if (jr >= scalar_load(p.plan + 2)) return;
  const int u_begin = jr * chunk;
  const int n_units = min(chunk, total - u_begin);

  // Position in the unit sequence: sequence b, page `page` of its run of R pages that
  // starts at unit U; L is the sequence's key length.
  struct Cursor { int b, page, R, U, L; };
  auto cursor_at = [&](int b, int u) __attribute__((always_inline)) {
    Cursor c;
    c.b = b;
    c.L = min(max(scalar_load(p.seqlens_k + b), 0), p.max_seqlen_k);
    c.R = (c.L + kPage - 1) / kPage;
    c.U = scalar_load(p.prefix + b);
    c.page = u - c.U;
    return c;
  };
  // Step to the next unit; only called while another unit remains in the range, so a
  // non-empty run follows.
  auto advance = [&](Cursor& c) __attribute__((always_inline)) {
    if (++c.page == c.R) {
      c.U += c.R;
      c.page = 0;
      do {
        ++c.b;
        c.L = min(max(scalar_load(p.seqlens_k + c.b), 0), p.max_seqlen_k);
        c.R = (c.L + kPage - 1) / kPage;
      } while (c.R == 0);
    }
  };

  const int64_t rs = (int64_t)p.hkv * D;     // elements between key rows of a page
  const int r_in = lane / CPR, pc = lane % CPR;
  uint32_t dma_off[NIW];
#pragma unroll
  for (int k = 0; k < NIW; ++k) {
    const int row = (wave * NIW + k) * RPI + r_in;
    dma_off[k] = (uint32_t)((row * rs + ((pc ^ dswz<D>(row)) << 3)) * 2);
  }
  int q_row[QIW], q_off[QIW];   // Q block row and element offset of this lane's copies
#pragma unroll
  for (int k = 0; k < QIW; ++k) {
    q_row[k] = (wave * QIW + k) * RPI + r_in;
    q_off[k] = (pc ^ dswz<D>(q_row[k])) << 3;
  }
  const uint32_t ring_base = lds_addr(ring);
  uint32_t page_ok_bits = 0;   // bit (local unit index mod 32): the page id was valid

  // Start the copies of unit `k` (local index) at cursor c into stage `stage`.
  // Page id of the unit at cursor c; read one issue ahead of its use so that the scalar
  // load's wait is not on the path from a barrier to the next copies.
  auto page_id = [&](const Cursor& c) __attribute__((always_inline)) {
    return scalar_load(p.block_table + (int64_t)c.b * p.max_blocks + c.page);
  };
  auto issue = [&](int k, const Cursor& c, int stage, int pg) __attribute__((always_inline)) {
    const bool page_ok = pg >= 0 && pg < p.num_blocks;
    page_ok_bits = (page_ok_bits & ~(1u << (k & 31))) | ((uint32_t)page_ok << (k & 31));
    const int64_t base = (int64_t)(page_ok ? pg : 0) * kPage * rs + (int64_t)kvh * D;
    const int key0 = c.page * kPage;
    const uint32_t ks = ring_base + stage * STAGE_B;
    const uint32_t vs = ks + TILE_B;
    const uint32_t qs = vs + TILE_B;
    if (page_ok && key0 + kPage <= c.L) {
#pragma unroll
      for (int i = 0; i < NIW; ++i) dma16_s<true>(p.k + base, dma_off[i], ks + (wave * NIW + i) * 1024);
#pragma unroll
      for (int i = 0; i < NIW; ++i) dma16_s<true>(p.v + base, dma_off[i], vs + (wave * NIW + i) * 1024);
    } else {
#pragma unroll
      for (int i = 0; i < NIW; ++i) {
        const bool ok = page_ok && key0 + (wave * NIW + i) * RPI + r_in < c.L;
        dma16_v<true>(ok ? p.k + base + dma_off[i] / 2 : kZeroChunk, ks + (wave * NIW + i) * 1024);
      }
#pragma unroll
      for (int i = 0; i < NIW; ++i) {
        const bool ok = page_ok && key0 + (wave * NIW + i) * RPI + r_in < c.L;
        dma16_v<true>(ok ? p.v + base + dma_off[i] / 2 : kZeroChunk, vs + (wave * NIW + i) * 1024);
      }
    }
    const uint16_t* qb = p.q + ((int64_t)c.b * p.hq + (int64_t)kvh * G) * D;
#pragma unroll
    for (int i = 0; i < QIW; ++i)
      dma16_v(q_row[i] < G ? qb + q_row[i] * D + q_off[i] : kZeroChunk, qs + (wave * QIW + i) * 1024);
  };

  // per-lane LDS read offsets inside a stage
  uint32_t koff[KS];
  uint32_t qoff[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    koff[s] = (16 * wave + lr) * ROWB + (((4 * s + lg) ^ dswz<D>(16 * wave + lr)) << 4);
    qoff[s] = 2 * TILE_B + lr * ROWB + (((4 * s + lg) ^ dswz<D>(lr)) << 4);
  }
  uint32_t voff[DB];
  {
    const int row = 16 * wave + 4 * lg + (lr >> 2);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int chunk_i = 2 * db + ((lr & 3) >> 1);
      voff[db] = TILE_B + row * ROWB + ((chunk_i ^ dswz<D>(row)) << 4) + 8 * (lr & 1);
    }
  }

  float m = -INFINITY, lsum = 0.f;   // state of query head lr over this wave's keys (log2)
  float4v acc[DB];                   // O^T: lane holds d = 16*db + 4*lg + i of head lr
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = float4v{0.f, 0.f, 0.f, 0.f};

  const int b_first = scalar_load(p.start + jr);
  Cursor ic = cursor_at(b_first, u_begin);   // next unit to copy
  int ipg = page_id(ic);                     // its page id
  Cursor cc = ic;                            // unit being consumed
  int piece_u0 = u_begin;                    // first unit of the current partition

  int istage = 0;
  const int pro = min(NST - 1, n_units);
  for (int k = 0; k < pro; ++k) {
    issue(k, ic, istage, ipg);
    istage = istage + 1 == NST ? 0 : istage + 1;
    if (k + 1 < n_units) {
      advance(ic);
      ipg = page_id(ic);
    }
  }

  // End of a partition whose last unit sits in `stage` (consumed by every wave): merge the
  // four waves' states through that stage, write the partial of run c to its slot and
  // restart the state empty.
  auto finish = [&](int stage, const Cursor& c, bool run_end) __attribute__((always_inline)) {
    const float l_w = rows4_sum(lsum);
    __syncthreads();
    float* mb = reinterpret_cast<float*>(ring + stage * STAGE_B);
    float* m_lds = mb + 3 * DB * 256;
    float* l_lds = m_lds + 3 * 64;
    if (wave > 0) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
        *reinterpret_cast<float4v*>(mb + (((wave - 1) * DB + db) * 64 + lane) * 4) = acc[db];
      m_lds[(wave - 1) * 64 + lane] = m;
      l_lds[(wave - 1) * 64 + lane] = l_w;
    }
    __syncthreads();
    if (wave == 0) {
      float mw[4], lw[4];
      mw[0] = m;
      lw[0] = l_w;
#pragma unroll
      for (int w = 1; w < 4; ++w) {
        mw[w] = m_lds[(w - 1) * 64 + lane];
        lw[w] = l_lds[(w - 1) * 64 + lane];
      }
      const float M = fmaxf(fmaxf(mw[0], mw[1]), fmaxf(mw[2], mw[3]));
      float sc[4], den = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        sc[w] = mw[w] == -INFINITY ? 0.f : fast_exp2(mw[w] - M);
        den += sc[w] * lw[w];
      }
      const float inv = den > 0.f ? 1.f / den : 0.f;
      const int slot = piece_u0 / chunk - c.U / chunk;
      const int64_t row0 = ((int64_t)c.b * p.hq + (int64_t)kvh * G) * S;
      if (lr < G) {
        const int64_t row = row0 + (int64_t)lr * S + slot;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          float4v o = acc[db] * sc[0];
#pragma unroll
          for (int w = 1; w < 4; ++w)
            o += *reinterpret_cast<const float4v*>(mb + (((w - 1) * DB + db) * 64 + lane) * 4) * sc[w];
          *reinterpret_cast<float4v*>(p.part_o + row * D + 16 * db + 4 * lg) = o * inv;
        }
        if (lg == 0) p.part_lse[row] = den > 0.f ? (M + __log2f(den)) * kLn2 : -INFINITY;
      }
      if (run_end)   // unused partitions of the run
        for (int e = lane; e < G * S; e += 64) {
          const int g = e / S, sl = e % S;
          if (sl > slot) p.part_lse[row0 + (int64_t)g * S + sl] = -INFINITY;
        }
    }
    m = -INFINITY;
    lsum = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] = float4v{0.f, 0.f, 0.f, 0.f};
  };

  int cstage = 0;
  if constexpr (!kPairs) {
    for (int i = 0; i < n_units; ++i) {
      wait_pages<PER, NST - 2>(min(NST - 2, n_units - 1 - i));
      __syncthreads();   // unit i visible to every wave; the stage of unit i - 1 is free
      if (i + NST - 1 < n_units) {
        issue(i + NST - 1, ic, istage, ipg);
        istage = istage + 1 == NST ? 0 : istage + 1;
        if (i + NST < n_units) {
          advance(ic);
          ipg = page_id(ic);
        }
      }

      const char* st = ring + cstage * STAGE_B;
      float4v s = {0.f, 0.f, 0.f, 0.f};   // S^T: keys 16*wave + 4*lg + j of the page, head lr
#pragma unroll
      for (int k = 0; k < KS; ++k)
        s = Op<T>::mfma(as_op<T>(*reinterpret_cast<const u32x4*>(st + koff[k])),
                        as_op<T>(*reinterpret_cast<const u32x4*>(st + qoff[k])), s);

      const bool page_ok = (page_ok_bits >> (i & 31)) & 1u;
      const int key = cc.page * kPage + 16 * wave + 4 * lg;
      float x[4];
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[j] = page_ok && key + j < cc.L ? s[j] * p.scale_log2 : -INFINITY;
        mx = fmaxf(mx, x[j]);
      }
      float alpha;
      const float m_use = move_ref(m, mx, alpha);
      float pr[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) pr[j] = fast_exp2(x[j] - m_use);
      const u32x2 pb = u32x2{pack2<T>(pr[0], pr[1]), pack2<T>(pr[2], pr[3])};
      lsum = Op<T>::sum2(pb[1], Op<T>::sum2(pb[0], lsum * alpha));
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const u32x2 a = lds_read_tr16(reinterpret_cast<const uint16_t*>(st + voff[db]));
        acc[db] = Op<T>::mfma16k(a, pb, acc[db] * alpha);
      }

      const bool run_end = cc.page == cc.R - 1;
      if (run_end || i == n_units - 1) {
        finish(cstage, cc, run_end);
        piece_u0 = u_begin + i + 1;
      }
      cstage = cstage + 1 == NST ? 0 : cstage + 1;
      if (i + 1 < n_units) advance(cc);
    }
  } else {
    // d = 64: a page holds half the bytes of a d = 128 page but its consumption is the same
    // chain of dependent steps (LDS reads, products, cross-lane max, exponentials, products),
    // which one wave per SIMD cannot hide. Two pages of one partition are therefore taken
    // per barrier, as one 128-key tile with the two chains interleaved; a unit that ends a
    // run alone is paired with itself, its second half masked out.
    int issued = pro;   // units whose copies have been started
    for (int i = 0; i < n_units;) {
      const bool two = i + 1 < n_units && cc.page + 1 < cc.R;
      const int c = two ? 2 : 1;
      wait_pages<PER, NST - 2>(issued - i - c);
      __syncthreads();   // units i .. i + c - 1 visible; the stages of earlier units are free
#pragma unroll
      for (int r = 0; r < 2; ++r)
        if (issued < n_units && issued - i < NST) {
          issue(issued, ic, istage, ipg);
          istage = istage + 1 == NST ? 0 : istage + 1;
          if (++issued < n_units) {
            advance(ic);
            ipg = page_id(ic);
          }
        }

      const char* sa = ring + cstage * STAGE_B;
      const char* sb = two ? ring + (cstage + 1 == NST ? 0 : cstage + 1) * STAGE_B : sa;
      float4v s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < KS; ++k) {
        const auto q = as_op<T>(*reinterpret_cast<const u32x4*>(sa + qoff[k]));
        s0 = Op<T>::mfma(as_op<T>(*reinterpret_cast<const u32x4*>(sa + koff[k])), q, s0);
        s1 = Op<T>::mfma(as_op<T>(*reinterpret_cast<const u32x4*>(sb + koff[k])), q, s1);
      }

      const bool ok0 = (page_ok_bits >> (i & 31)) & 1u;
      const bool ok1 = two && ((page_ok_bits >> ((i + 1) & 31)) & 1u);
      const int key = cc.page * kPage + 16 * wave + 4 * lg;
      float x[8];
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[j] = ok0 && key + j < cc.L ? s0[j] * p.scale_log2 : -INFINITY;
        x[4 + j] = ok1 && key + kPage + j < cc.L ? s1[j] * p.scale_log2 : -INFINITY;
        mx = fmaxf(mx, fmaxf(x[j], x[4 + j]));
      }
      float alpha;
      const float m_use = move_ref(m, mx, alpha);
      float pr[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) pr[j] = fast_exp2(x[j] - m_use);
      const u32x2 pb0 = u32x2{pack2<T>(pr[0], pr[1]), pack2<T>(pr[2], pr[3])};
      const u32x2 pb1 = u32x2{pack2<T>(pr[4], pr[5]), pack2<T>(pr[6], pr[7])};
      lsum = Op<T>::sum2(pb1[1], Op<T>::sum2(pb1[0], Op<T>::sum2(pb0[1], Op<T>::sum2(pb0[0], lsum * alpha))));
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const u32x2 a0 = lds_read_tr16(reinterpret_cast<const uint16_t*>(sa + voff[db]));
        const u32x2 a1 = lds_read_tr16(reinterpret_cast<const uint16_t*>(sb + voff[db]));
        acc[db] = Op<T>::mfma16k(a1, pb1, Op<T>::mfma16k(a0, pb0, acc[db] * alpha));
      }

      const bool run_end = cc.page + c - 1 == cc.R - 1;
      if (run_end || i + c == n_units) {
        finish(cstage, cc, run_end);
        piece_u0 = u_begin + i + c;
      }
      cstage = cstage + c >= NST ? cstage + c - NST : cstage + c;
      if (i + 1 < n_units) advance(cc);
      if (two && i + 2 < n_units) advance(cc);
      i += c;
    }
  }
}

// One wave per (sequence, head), or per query row of a prefill tail split (row map):
// lane s holds split s's lse.
template <int D>
__global__ __launch_bounds__(kThreads) void combine_kernel(const CombineParams p) {
  constexpr int PER = D / 64;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int pair = blockIdx.x * kWaves + wave;
  if (pair >= p.pairs) return;
  const int S = p.num_splits;
  int64_t obase = (int64_t)pair * D, li = pair;
  if (p.row_off) {
    obase = p.row_off[pair];
    if (obase < 0) return;                          // padding row of a work item
    li = p.row_lse[pair];
  }
  if (p.seqlens_k && min(scalar_load(p.seqlens_k + pair / p.heads), p.max_seqlen_k) <= 0) {
    // a sequence with no key: no partial was written for it
    const int64_t ob = obase + lane * PER;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      if (p.o_dtype == kF32) static_cast<float*>(p.o)[ob + e] = 0.f;
      else static_cast<uint16_t*>(p.o)[ob + e] = 0;
    }
    if (p.lse && lane == 0 && li >= 0) p.lse[li] = -INFINITY;
    return;
  }
  const float l = lane < S ? p.part_lse[(int64_t)pair * S + lane] : -INFINITY;
  float M = l;
#pragma unroll
  for (int msk = 1; msk < 64; msk <<= 1) M = wave_max_xor(M, msk);
  const float w = (M == -INFINITY || l == -INFINITY) ? 0.f : fast_exp2((l - M) * kLog2e);
  float den = w;
#pragma unroll
  for (int msk = 1; msk < 64; msk <<= 1) den = wave_sum_xor(den, msk);

  // The partials of CH splits are loaded together, so that their latencies overlap
  // (a load per split behind a branch on its weight would wait for each in turn). A split
  // of weight 0 (no key; its O_s may never have been written) is read like the others,
  // inside the workspace, and then left out by a select, so the sum is the same, term by
  // term and in the same order, as skipping it.
  constexpr int CH = 8;
  float o[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) o[e] = 0.f;
  for (int s0 = 0; s0 < S; s0 += CH) {
    float v[CH][PER], ws[CH];
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      const int s = min(s0 + k, S - 1);
      ws[k] = s0 + k < S ? __shfl(w, s, 64) : 0.f;
      const float* src = p.part_o + ((int64_t)pair * S + s) * D + lane * PER;
#pragma unroll
      for (int e = 0; e < PER; ++e) v[k][e] = src[e];
    }
#pragma unroll
    for (int k = 0; k < CH; ++k)
#pragma unroll
      for (int e = 0; e < PER; ++e) o[e] = ws[k] != 0.f ? fmaf(ws[k], v[k][e], o[e]) : o[e];
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  const int64_t ob = obase + lane * PER;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const float v = o[e] * inv;
    if (p.o_dtype == kF32) static_cast<float*>(p.o)[ob + e] = v;
    else if (p.o_dtype == kF16) static_cast<uint16_t*>(p.o)[ob + e] = Op<F16>::from_float(v);
    else static_cast<uint16_t*>(p.o)[ob + e] =
        p.o_round == 0 ? Op<BF16>::from_float(v) : (uint16_t)bf16_bits_directed(v, p.o_round);
  }
  if (p.lse && lane == 0 && li >= 0) p.lse[li] = den > 0.f ? M + __logf(den) : -INFINITY;
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

template <int D, typename T>
hipError_t launch_stream_t(const DecodeParams& p, hipStream_t s) {
  hipLaunchKernelGGL(decode_plan_kernel, dim3(1), dim3(1024), 0, s, p);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_stream_kernel<D, T, kStreamStages<D>>), dim3(p.nwk * p.hkv), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_stream_d(const DecodeParams& p, int qkv_dtype, hipStream_t s) {
  return qkv_dtype == kF16 ? launch_stream_t<D, F16>(p, s) : launch_stream_t<D, BF16>(p, s);
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

hipError_t launch_decode_stream(const DecodeParams& p, int head_dim, int qkv_dtype,
                                hipStream_t stream) {
  switch (head_dim) {
    case 64: return launch_stream_d<64>(p, qkv_dtype, stream);
    case 128: return launch_stream_d<128>(p, qkv_dtype, stream);
    case 256: return launch_stream_d<256>(p, qkv_dtype, stream);
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
