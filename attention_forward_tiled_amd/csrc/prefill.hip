// Tiled attention forward (prefill) for gfx950.
//
// What is computed: the online-softmax recurrence of the page "gfx942 unified
// attention, from the math up", section 3 (running max m, denominator l and
// un-normalised output o per query row, O = o / l at the end), over 64-key tiles, with
// the bottom-right causal mask and early exit of section 4 and the paged K/V gather of
// section 5. Scores are handled in the base-2 domain (s * tau * log2 e, exp2).
//
// How it is mapped onto CDNA4:
//   * A group of NW waves owns 32 * NW query rows that share one KV head: for a GQA
//     group of G query heads it takes 32 * NW / G positions of every head of the group,
//     so each K/V tile brought into LDS serves all G heads. Three launch forms (chosen
//     on the host, see launch_one): eight waves / 256 rows for large launches at
//     d = 128 (twice the rows per copied tile); two groups of four waves splitting one
//     block's key tiles (merged through LDS) for causal launches with few blocks,
//     optionally pairing a heavy and a light block per workgroup; otherwise four waves /
//     128 rows, two workgroups per CU (three at d = 64).
//   * Each wave owns 32 rows. Scores are produced transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16: K comes from LDS as the A operand and Q stays in registers
//     as the B operand for the whole kernel. The accumulator then holds, per lane, one
//     query row and 32 of the tile's keys (the other 32 sit in lane l ^ 32), which is
//     exactly the B-operand layout the P.V product needs, so P never leaves registers.
//     The 32x32x16 atom (rather than 16x16x32) leaves more issue slots to the softmax
//     VALU work of the other wave on the same SIMD and halves the MFMA count.
//   * O^T += V^T P^T with the same MFMA; the V^T operand is read from the row-major
//     V tile with ds_read_b64_tr_b16, which transposes 4x4 blocks of 16-bit values
//     on the way out of LDS. K and V are therefore stored in LDS exactly as they sit
//     in memory (row-major, 16-byte chunks XOR-swizzled by row to spread banks), and
//     are copied there by global_load_lds_dwordx4 without passing through registers.
//   * Two LDS stages: tile j+1 is in flight while tile j is consumed; one barrier per
//     tile. The main loop is unrolled by two so every LDS offset is an immediate. In
//     the eight-wave form one wave per SIMD issues the copies (the address unit takes
//     them one at a time; the SIMD's other wave meanwhile starts its products).
//   * Tiles entirely inside the visible region run a loop with no masking code; the
//     tiles that straddle the causal diagonal or the key length run a second loop that
//     masks scores and fetches rows past the key length from a block of zeros (NaN in
//     unused page slots never meets a zero probability in P.V).
//   * The reference maximum behind o and l moves lazily: only when a row's maximum
//     exceeds it by more than 2^8, so the O rescale is skipped on most tiles; each lane
//     tests its own scores first, so most tiles also skip the cross-lane max exchange.
//   * Row sums of P are taken from the packed 16-bit P with v_dot2 (the same values
//     the P.V MFMA consumes).
//   * The workgroup order is reversed over query blocks so that, under a causal
//     mask, the longest-running blocks are dispatched first.
//   * d = 256 runs prefill_narrow_kernel instead: eight waves of 16 rows, two per SIMD
//     (32 rows of d = 256 would need about 500 registers, one wave per SIMD).
//   * Tail split (host: plan_one): when the last round of a non-causal launch, or a whole
//     causal launch of few items, would leave at least half of the CUs idle, the key
//     tiles of those items are cut into parts, one one-group workgroup per (item, part);
//     each part writes its normalised fp32 O and lse, and the log-sum-exp combine of
//     section 8 of the same page merges them into O through a row map.
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace attn {

namespace {

constexpr float kLazy = 8.0f;          // log2-domain slack before the reference max moves

// 16-byte chunk swizzle, chunk' = chunk ^ swz(row). It must spread two read patterns
// over the 64 banks: the K reads (16 consecutive rows at one chunk per 16 lanes) and the
// V transpose reads (4 consecutive rows x 4 consecutive chunks per 32 lanes). Rotating
// the low row bits before the XOR serves both: for d >= 128 (256-byte rows) the low
// four row bits are rotated by two; for d = 64 (two rows per 256 bytes) the three bits
// above the row's parity are rotated by one. Only row % 16 (row % 32 for d = 64)
// matters, so rows 16 or 32 apart share a pattern.
template <int D>
__device__ __forceinline__ int swz(int row) {
  if constexpr (D == 64) {
    const int k = (row >> 1) & 7;
    return ((k & 1) << 2) | (k >> 1);
  } else {
    const int r = row & 15;
    return ((r & 3) << 2) | (r >> 2);
  }
}

// NG groups of NW waves per workgroup; a group owns 32 * NW query rows. With NG = 2 (NW = 4)
// both groups own the same 128 query rows and split the workgroup's key tiles between
// them, merging their (o, m, l) at the end; this halves the longest workgroup when there
// are too few workgroups to balance the causal triangle. Each group has its own two LDS
// stages. With NW = 8 (NG = 1) eight waves share every K/V tile copied to LDS, which
// halves the copy traffic per query row on large launches. With PAIR, a workgroup
// processes two query blocks of one (sequence, KV head) in turn (see below).
template <int D, int NG, int NW, typename T, bool PRECISE, bool PAIR>
__global__ __launch_bounds__(64 * NW * NG, D == 256 ? 1 : 2)
void prefill_kernel(const PrefillParams p) {
  constexpr int KS = D / 16;            // k-steps (16 deep) of the S^T product
  constexpr int DB = D / 32;            // 32-wide d blocks of O^T
  constexpr int CPR = D / 8;            // 16-byte chunks per row
  constexpr int RPI = 512 / D;          // rows covered by one 1 KiB wave-wide LDS copy
  constexpr int NIW = kPage / RPI / NW;   // such copies per wave per tile (K and V each)
  constexpr int TILE = kPage * D;       // elements per K (or V) tile
  constexpr int ROWB = D * 2;           // bytes per LDS row
  __shared__ __align__(16) uint16_t smem[NG * 2 * 2 * TILE];   // [group][2 stages][K, V][TILE]
  if constexpr (kPoisonLds) poison_lds<sizeof(smem)>(smem);

  const int tid = threadIdx.x, lane = tid & 63;
  const int grp = tid / (64 * NW);                              // key-range group
  const int wave = (tid >> 6) % NW;                            // wave inside it
  const int lq = lane & 31, half = lane >> 5;        // query column, k-half of the 32x32 layouts

  // The dispatcher hands workgroups to the 8 XCDs round-robin. Workgroup x is given work
  // item `lid` so that each XCD walks a contiguous run of items: the query blocks of one
  // (sequence, KV head) in a row, heaviest (last) first. Workgroups resident on an XCD at
  // the same time then stream the same K/V through its L2, and the longest causal blocks
  // start first.
  const int nx = gridDim.x, xcd = blockIdx.x & 7, per = nx >> 3, extra = nx & 7;
  const int lid = xcd * per + min(xcd, extra) + (int)(blockIdx.x >> 3);
  const int nq = (p.seqlen_q + p.bq - 1) / p.bq;
  // In a tail-split launch, `lid` numbers (item, key part) units, the parts of an item
  // next to each other.
  constexpr bool CAN_SPLIT = NG == 1 && !PAIR && !PRECISE;   // the forms a tail split uses
  const int nsp = CAN_SPLIT ? p.split_parts : 0;
  const int item = nsp ? p.split_item0 + lid / nsp : lid;
  const int part = nsp ? lid % nsp : 0;
  // With pairing, a workgroup takes query blocks nq - 1 - u and u of one (sequence, KV
  // head) one after the other; under a causal mask their tile counts add up to about the
  // same total for every u.
  const int nu = PAIR ? (nq + 1) / 2 : nq;
  const int unit = item % nu;
  const int bh = item / nu;
  const int b = bh % p.batch, kvh = bh / p.batch;

  int L = p.seqlen_k;
  if (p.seqlens_k) L = min(max(scalar_load(p.seqlens_k + b), 0), p.seqlen_k);
  // Queries of this sequence: S_q rows from row qrow0 (packed queries: the sequence's
  // own count and first row in the shared buffer).
  int sq = p.seqlen_q;
  int64_t qrow0 = 0;
  if (p.cu_seqlens_q) {
    const int c0 = scalar_load(p.cu_seqlens_q + b);
    sq = min(max(scalar_load(p.cu_seqlens_q + b + 1) - c0, 0), p.seqlen_q);
    qrow0 = c0;
  }
  const int off = L - sq;               // bottom-right alignment of the causal mask
  const float c = p.scale_log2;

  // state of the current query block (set at the start of each item)
  int q0 = 0, rpos = 0, rh = 0, n_full = 0, h = 0, j0 = 0, j1 = 0;
  bool rok = false;
  u32x4 qf[KS];

  // ---- per-lane constants of the K/V copies (byte offsets inside a tile's rows)
  const bool paged = p.block_table != nullptr;
  const int64_t rs = paged ? (int64_t)p.hkv * D : p.kv_ss;   // elements between key rows
  const int r_in = lane / CPR, pc = lane % CPR;
  // Eight-wave form: waves 0-3 (one per SIMD) copy the rows of wave pairs (2w, 2w+1), so
  // that on every SIMD one wave starts its products while the other issues copies.
  constexpr int CW = NW == 8 ? 2 : 1;          // copy shares per issuing wave
  const int cw0 = NW == 8 ? 2 * (wave & 3) : wave;
  uint32_t dma_off[CW][NIW];
#pragma unroll
  for (int v = 0; v < CW; ++v)
#pragma unroll
    for (int k = 0; k < NIW; ++k) {
      const int row = ((cw0 + v) * NIW + k) * RPI + r_in;
      dma_off[v][k] = (uint32_t)((row * rs + ((pc ^ swz<D>(row)) << 3)) * 2);
    }
  // this lane's Q fragments (B operand of S^T) for the rows set by rpos, rh, rok
  auto load_q = [&]() {
    const uint16_t* qp = p.q + b * p.q_sb + (int64_t)rh * p.q_sh + (qrow0 + rpos) * p.q_ss;
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = rok ? ldg16(qp + s * 16 + half * 8) : u32x4{0, 0, 0, 0};
  };

  const uint32_t smem_base = lds_addr(smem) + grp * 2 * 2 * TILE * 2;
  // The group's byte offset is folded into the per-lane read offsets below, so that
  // the stage bases stay compile-time constants (immediate offsets of the LDS reads).
  const uint32_t goff = grp * 2 * 2 * TILE * 2;

  // Copy tile j into this group's LDS stage `stage`. Rows past the key length, and every
  // row of a page whose id is out of range, are fetched from the zero block instead; the
  // keys of such a page are left out altogether (bit `stage` of stage_ok is cleared and
  // the tile is skipped), as in the decode kernels.
  uint32_t stage_ok = 3u;
  auto issue_tile = [&](int j, int stage) {
    int64_t base;
    bool page_ok = true;
    if (paged) {
      // j is wave-uniform: say so, so that the page id comes in by a scalar load, which
      // leaves the vector-memory counter to the tile copies
      const int pg = scalar_load(p.block_table + (int64_t)b * p.max_blocks + __builtin_amdgcn_readfirstlane(j));
      page_ok = pg >= 0 && pg < p.num_blocks;
      base = (int64_t)(page_ok ? pg : 0) * kPage * p.hkv * D + (int64_t)kvh * D;
    } else {
      base = b * p.kv_sb + kvh * p.kv_sh + (int64_t)j * kPage * p.kv_ss;
    }
    stage_ok = page_ok ? (stage_ok | (1u << stage)) : (stage_ok & ~(1u << stage));
    const uint32_t ks = smem_base + stage * 2 * TILE * 2;
    const uint32_t vs = ks + TILE * 2;
    if (NW == 8 && wave >= 4) return;
    if (page_ok && (j + 1) * kPage <= L) {
#pragma unroll
      for (int v = 0; v < CW; ++v)
#pragma unroll
        for (int k = 0; k < NIW; ++k) {
          const int i = (cw0 + v) * NIW + k;
          dma16_s(p.k + base, dma_off[v][k], ks + i * 1024);
          dma16_s(p.v + base, dma_off[v][k], vs + i * 1024);
        }
    } else {
#pragma unroll
      for (int v = 0; v < CW; ++v)
#pragma unroll
        for (int k = 0; k < NIW; ++k) {
          const int i = (cw0 + v) * NIW + k;
          const bool ok = page_ok && (j * kPage + (i * RPI + r_in) < L);
          dma16_v(ok ? p.k + base + dma_off[v][k] / 2 : kZeroChunk, ks + i * 1024);
          dma16_v(ok ? p.v + base + dma_off[v][k] / 2 : kZeroChunk, vs + i * 1024);
        }
    }
  };

  // ---- per-lane LDS read offsets (bytes inside a stage's K or V tile)
  // K A-operand for S^T: row 32*kb + lq (kb enters as an immediate), chunk 2*s + half.
  uint32_t koff[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) koff[s] = goff + lq * ROWB + (((2 * s + half) ^ swz<D>(lq)) << 4);
  // V^T A-operand via transpose reads: lane (g = lane/16, j = lane%16) addresses row
  // 16*t + 8*h + 4*(g/2) + j/4 (t enters as an immediate) at column 32*db + 16*(g%2) + 4*(j%4).
  const int tg = lane >> 4, tj = lane & 15;
  uint32_t voff[2][DB];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int row = 8 * hh + 4 * (tg >> 1) + (tj >> 2);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int col = 32 * db + 16 * (tg & 1) + 4 * (tj & 3);
      voff[hh][db] = goff + row * ROWB + (((col >> 3) ^ swz<D>(row)) << 4) + (col & 7) * 2;
    }
  }

  float mref = -INFINITY;   // reference max (log2 domain) behind o and l
  float lsum = 0.f;         // this lane's share of l (its 32 keys of each tile)
  float16v acc[DB];

  // One tile from stage STAGE of this group: S^T = K Q^T, online softmax, O^T += V^T P^T.
  auto compute = [&](int j, auto stage_c, auto mask_c, auto&& mid) {
    constexpr int STAGE = decltype(stage_c)::value;
    constexpr bool MASK = decltype(mask_c)::value;
    const char* ks = reinterpret_cast<const char*>(smem) + STAGE * 2 * TILE * 2;
    const char* vs = ks + TILE * 2;

    // scores of keys 32*kb + 8*g + 4*half + i, at sc[kb][4*g + i]
    float16v sc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sc[kb] = float16v{};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(ks + koff[s] + kb * 32 * ROWB);
        sc[kb] = Op<T>::mfma32(as_op<T>(a), as_op<T>(qf[s]), sc[kb]);
      }
    }

    mid();   // (the two-group form's group 1 issues its next tile here)

    if constexpr (MASK) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = j * kPage + 32 * kb + 8 * (e >> 2) + 4 * half + (e & 3);
          const bool vis = key < L && (!p.causal || key <= rpos + off);
          sc[kb][e] = vis ? sc[kb][e] : -INFINITY;
        }
    }

    // Online softmax with a lazily moved reference maximum: o and l are kept relative to
    // mref, which only moves (rescaling o and l by 2^(old - new)) when the row maximum
    // exceeds it by more than kLazy, so every p stays <= 2^kLazy. A lane first checks its
    // own 32 scores (a shallow max tree, no cross-lane exchange); only when some lane sees
    // a score above the slack is the row maximum formed across the two lanes of each row.
    float m8[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float16v& x = sc[i >> 2];
      const int e = 4 * (i & 3);
      m8[i] = fmaxf(fmaxf(x[e], x[e + 1]), fmaxf(x[e + 2], x[e + 3]));
    }
    const float mx = fmaxf(fmaxf(fmaxf(m8[0], m8[1]), fmaxf(m8[2], m8[3])),
                           fmaxf(fmaxf(m8[4], m8[5]), fmaxf(m8[6], m8[7])));
    if (__builtin_amdgcn_ballot_w64(mx * c > mref + kLazy) != 0) {
      const float mt = wave_max_xor(mx, 32) * c;
      const bool up = mt > mref + kLazy;
      const float nref = up ? mt : mref;
      const float alpha = up ? fast_exp2(mref - nref) : 1.f;
      mref = nref;
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[db] *= alpha;
    }

    const float mneg = mref == -INFINITY ? 0.f : -mref;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) sc[kb][e] = fast_exp2(__builtin_fmaf(sc[kb][e], c, mneg));

    // P^T B-operand of key step t (keys 16t..16t+15): elements 8*(t%2) .. +7 of sc[t/2]
    u32x4 pf[4];
    u32x4 pl[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const float16v& x = sc[t >> 1];
      const int e0 = 8 * (t & 1);
      pf[t] = u32x4{pack2<T>(x[e0], x[e0 + 1]), pack2<T>(x[e0 + 2], x[e0 + 3]),
                    pack2<T>(x[e0 + 4], x[e0 + 5]), pack2<T>(x[e0 + 6], x[e0 + 7])};
      if constexpr (PRECISE) {
        float rr[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) rr[i] = x[e0 + i] - Op<T>::to_float(Op<T>::from_float(x[e0 + i]));
        pl[t] = u32x4{pack2<T>(rr[0], rr[1]), pack2<T>(rr[2], rr[3]),
                      pack2<T>(rr[4], rr[5]), pack2<T>(rr[6], rr[7])};
      }
    }
    if constexpr (PRECISE) {
      float ps = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) ps += sc[kb][e];
      lsum += ps;
    } else {
      float ps0 = lsum, ps1 = 0.f;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        ps0 = Op<T>::sum2(pf[t][0], ps0);
        ps1 = Op<T>::sum2(pf[t][1], ps1);
        ps0 = Op<T>::sum2(pf[t][2], ps0);
        ps1 = Op<T>::sum2(pf[t][3], ps1);
      }
      lsum = ps0 + ps1;
    }

#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const u32x2 lo = lds_read_tr16(reinterpret_cast<const uint16_t*>(vs + voff[0][db] + 16 * t * ROWB));
        const u32x2 hi = lds_read_tr16(reinterpret_cast<const uint16_t*>(vs + voff[1][db] + 16 * t * ROWB));
        const u32x4 a = u32x4{lo[0], lo[1], hi[0], hi[1]};
        acc[db] = Op<T>::mfma32(as_op<T>(a), as_op<T>(pf[t]), acc[db]);
        if constexpr (PRECISE) acc[db] = Op<T>::mfma32(as_op<T>(a), as_op<T>(pl[t]), acc[db]);
      }
    }
  };

  using Full = std::integral_constant<bool, false>;
  using Masked = std::integral_constant<bool, true>;

  // Step i of the workgroup: both groups take their i-th tile in lockstep (one barrier per
  // step publishes the stage and recycles the other); a group whose range is exhausted
  // only joins the barriers.
  auto step = [&](int i, auto stage_c, auto mask_c) {
    constexpr int STAGE = decltype(stage_c)::value;
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
    const int j = j0 + i;
    // two-group form at d = 128: group 0 issues the next tile's copies now, group 1 after
    // its S^T products, so that on each SIMD one wave issues copies while the other
    // computes (+1 to +3% on the causal shapes of this form, bit-equal; at d = 64, with
    // half the products per tile, -1%)
    const bool late = NG == 2 && D == 128 && grp == 1;
    if (j + 1 < j1 && !late) issue_tile(j + 1, STAGE ^ 1);
    auto mid = [&]() { if (late && j + 1 < j1) issue_tile(j + 1, STAGE ^ 1); };
    if (((stage_ok >> STAGE) & 1u) && j < j1) compute(j, stage_c, mask_c, mid);
    else mid();
  };

  for (int it = 0; it < (PAIR ? 2 : 1); ++it) {
    const int qblk = it == 0 ? nq - 1 - unit : unit;
    if (it == 1 && qblk >= nq - 1 - unit) break;   // the middle block of an odd count
    q0 = qblk * p.bq;

    // ---- this lane's query row and its Q fragments (B operand of S^T); the second item's
    // fragments were requested before the first item's merge and store
    {
      const int r = wave * 32 + lq;
      const int hig = r / p.bq;
      rpos = q0 + (r - hig * p.bq);
      rh = kvh * p.group + hig;
      rok = hig < p.group && rpos < sq;
      if (it == 0) load_q();
    }

    // ---- tile range: [0, n_full) need no masking, [n_full, n_tiles) straddle a boundary;
    // group g takes tiles [g*h, min((g+1)*h, n_tiles)), h = ceil(n_tiles / NG)
    {
      const int pmax = min(q0 + p.bq, sq) - 1;
      const int kv_end = p.causal ? min(L, pmax + off + 1) : L;
      const int n_tiles = kv_end > 0 && q0 < sq ? (kv_end + kPage - 1) / kPage : 0;
      n_full = L / kPage;
      if (p.causal) n_full = min(n_full, max(q0 + off + 1, 0) / kPage);
      n_full = min(n_full, n_tiles);
      h = (n_tiles + NG - 1) / NG;
      j0 = grp * h;
      j1 = min(n_tiles, j0 + h);
      if (nsp) {
        // tail split (one group): this unit's share of the key tiles
        const int tp = (n_tiles + nsp - 1) / nsp;
        j0 = min(part * tp, n_tiles);
        j1 = min(n_tiles, j0 + tp);
        h = j1 - j0;
      }
    }

    mref = -INFINITY;
    lsum = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] = float16v{};

    if (j0 < j1) issue_tile(j0, 0);
    // steps [0, nf) take tiles that need no mask; the rest take masked tiles or (a group
    // whose range is exhausted) only join the barriers. Two loops, one kind of tile body
    // each, so that each keeps one register assignment.
    const int nf = max(0, min(n_full, j1) - j0);
    int i = 0;
    for (; i + 1 < nf; i += 2) {
      step(i, std::integral_constant<int, 0>{}, Full{});
      step(i + 1, std::integral_constant<int, 1>{}, Full{});
    }
    if (i < nf) {
      step(i, std::integral_constant<int, 0>{}, Full{});
      ++i;
    }
    for (; i < h; ++i) {
      if (i & 1) step(i, std::integral_constant<int, 1>{}, Masked{});
      else step(i, std::integral_constant<int, 0>{}, Masked{});
    }

    if constexpr (PAIR) {
      // Q of the second item (the registers are free once the last tile is done): its
      // load overlaps this item's merge and store.
      if (it == 0 && unit < nq - 1 - unit) {
        const int r = wave * 32 + lq;
        const int hig = r / p.bq;
        const int pos = unit * p.bq + (r - hig * p.bq);
        const bool ok = hig < p.group && pos < sq;
        const uint16_t* qp = p.q + b * p.q_sb + (int64_t)(kvh * p.group + hig) * p.q_sh + (qrow0 + pos) * p.q_ss;
#pragma unroll
        for (int s = 0; s < KS; ++s) qf[s] = ok ? ldg16(qp + s * 16 + half * 8) : u32x4{0, 0, 0, 0};
      }
    }

    if constexpr (NG == 2) {
      // Hand group 1's (o, m, l) to group 0 through LDS and merge them there:
      // M = max(m0, m1), o = 2^(m0-M) o0 + 2^(m1-M) o1, l likewise.
      constexpr int STRIDE = (DB * 16 + 2) * 64;     // floats per wave
      float* xb = reinterpret_cast<float*>(smem) + wave * STRIDE + lane;
      __syncthreads();
      if (grp == 1) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int e = 0; e < 16; ++e) xb[(db * 16 + e) * 64] = acc[db][e];
        xb[DB * 16 * 64] = mref;
        xb[(DB * 16 + 1) * 64] = lsum;
      }
      __syncthreads();
      if (grp == 0) {
        const float m1 = xb[DB * 16 * 64];
        const float l1 = xb[(DB * 16 + 1) * 64];
        const float M = fmaxf(mref, m1);
        const float w0 = mref == -INFINITY ? 0.f : fast_exp2(mref - M);
        const float w1 = m1 == -INFINITY ? 0.f : fast_exp2(m1 - M);
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[db][e] = w0 * acc[db][e] + w1 * xb[(db * 16 + e) * 64];
        lsum = w0 * lsum + w1 * l1;
        mref = M;
      }
    }

    // ---- epilogue: O = o / l, lse = ln 2 * (mref + log2 l); lane holds d = 32*db + 8*g + 4*half + i
    const float l = wave_sum_xor(lsum, 32);
    // element offset of the row in o; its index in lse: [B, Hq, S_q], or [Hq, total_q] for
    // packed queries
    auto o_offset = [&]() { return b * p.o_sb + (int64_t)rh * p.o_sh + (qrow0 + rpos) * p.o_ss; };
    auto lse_index = [&]() {
      return p.cu_seqlens_q ? (int64_t)rh * scalar_load(p.cu_seqlens_q + p.batch) + qrow0 + rpos
                            : ((int64_t)b * p.hq + rh) * p.seqlen_q + rpos;
    };
    if (CAN_SPLIT && nsp) {
      // tail split: this part's normalised O and lse in fp32, for the combine; part 0 also
      // records where the row goes (-1 for a padding row)
      const int64_t prow = (int64_t)(lid / nsp) * (32 * NW) + wave * 32 + lq;
      if (rok) {
        const float inv = l > 0.f ? 1.f / l : 0.f;
        float* po = p.part_o + (prow * nsp + part) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g)
            *reinterpret_cast<float4v*>(po + 32 * db + 8 * g + 4 * half) =
                float4v{acc[db][4 * g], acc[db][4 * g + 1], acc[db][4 * g + 2], acc[db][4 * g + 3]} * inv;
        if (half == 0) p.part_lse[prow * nsp + part] = l > 0.f ? (mref + __log2f(l)) * kLn2 : -INFINITY;
      }
      if (half == 0 && part == 0) {
        p.row_off[prow] = rok ? o_offset() : -1;
        p.row_lse[prow] = rok && p.lse ? lse_index() : -1;
      }
    } else if (grp == 0 && rok) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const int64_t ob = o_offset();
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * db + 8 * g + 4 * half;
        const float4v v = float4v{acc[db][4 * g], acc[db][4 * g + 1], acc[db][4 * g + 2], acc[db][4 * g + 3]} * inv;
        if (p.o_dtype == kF32) {
          *reinterpret_cast<float4v*>(static_cast<float*>(p.o) + ob + d0) = v;
        } else if (p.o_dtype == kF16) {
          *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(p.o) + ob + d0) =
              u32x2{pack2<F16>(v[0], v[1]), pack2<F16>(v[2], v[3])};
        } else {
          *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(p.o) + ob + d0) =
              u32x2{pack_bf16_round(v[0], v[1], p.o_round), pack_bf16_round(v[2], v[3], p.o_round)};
        }
      }
    }
    if (p.lse && half == 0) p.lse[lse_index()] = l > 0.f ? (mref + __log2f(l)) * kLn2 : -INFINITY;
    }
    if constexpr (PAIR) __syncthreads();   // the LDS of this item is the next item's staging area
  }
}


// Narrow form for d = 256: eight waves, two per SIMD, 16 query rows per wave, 128 per
// workgroup. The 32-row form needs about 500 registers at d = 256 and so runs one wave per
// SIMD, which leaves every LDS and softmax latency exposed; with 16 rows a wave holds O^T
// in 64 registers. Products on the 16-wide atoms: S^T = K Q^T with v_mfma_f32_16x16x32
// (K from LDS as the A operand, Q in registers), O^T += V^T P^T with the same atom over 32
// keys (two 16-key blocks of the S^T accumulator, whose layout is the B-operand layout
// with the keys enumerated per block), so P stays in registers; V^T comes from the
// row-major V tile by transposed LDS reads. Waves 0-3 (one per SIMD) issue the tile copies. Lane l holds query row l % 16
// of its wave and keys 16 kb + 4 (l / 16) + i of every 16-key block kb; the other keys of
// the row sit in lanes l ^ 16, l ^ 32, l ^ 48. Chunks are swizzled by the 16-row pattern
// (qswz) that keeps both read patterns free of bank conflicts: chunk' = chunk ^ 2 (row % 16),
// so that the V^T reads of 8 rows x 2 chunks hit distinct banks and rows r and r + 8 of
// the K reads sit in different 256-byte halves of their 512-byte rows. (The rotation
// ((r & 7) << 1) | (r >> 3), which puts row bit 3 into chunk bit 0 instead, cost about
// 4 conflict cycles per K read on a probe of these two read patterns; every mask that
// sends row bit 3 to chunk bit 4 measured none for either pattern.)
template <int D>
__device__ __forceinline__ int qswz(int row) {
  return (row & 15) << 1;
}

template <int D, typename T>
__global__ __launch_bounds__(512, 1)
void prefill_narrow_kernel(const PrefillParams p) {
  constexpr int NW = 8;
  constexpr int KS = D / 32;            // k-steps (32 deep) of S^T
  constexpr int DB = D / 16;            // 16-wide d blocks of O^T
  constexpr int CPR = D / 8;            // 16-byte chunks per row
  constexpr int RPI = 512 / D;          // rows per 1 KiB wave-wide copy
  constexpr int NIW = kPage / RPI / NW; // such copies per wave per tile (K and V each)
  constexpr int TILE = kPage * D;
  constexpr int ROWB = D * 2;
  __shared__ __align__(16) uint16_t smem[2 * 2 * TILE];   // [2 stages][K, V][TILE]
  if constexpr (kPoisonLds) poison_lds<sizeof(smem)>(smem);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;

  const int nx = gridDim.x, xcd = blockIdx.x & 7, per = nx >> 3, extra = nx & 7;
  const int lid = xcd * per + min(xcd, extra) + (int)(blockIdx.x >> 3);
  const int nq = (p.seqlen_q + p.bq - 1) / p.bq;
  // tail split: `lid` numbers (item, key part) units, as in prefill_kernel
  const int nsp = p.split_parts;
  const int item = nsp ? p.split_item0 + lid / nsp : lid;
  const int part = nsp ? lid % nsp : 0;
  const int unit = item % nq;
  const int bh = item / nq;
  const int b = bh % p.batch, kvh = bh / p.batch;

  int L = p.seqlen_k;
  if (p.seqlens_k) L = min(max(scalar_load(p.seqlens_k + b), 0), p.seqlen_k);
  int sq = p.seqlen_q;
  int64_t qrow0 = 0;
  if (p.cu_seqlens_q) {
    const int c0 = scalar_load(p.cu_seqlens_q + b);
    sq = min(max(scalar_load(p.cu_seqlens_q + b + 1) - c0, 0), p.seqlen_q);
    qrow0 = c0;
  }
  const int off = L - sq;
  const float c = p.scale_log2;
  const int q0 = (nq - 1 - unit) * p.bq;

  // this lane's query row
  const int R = wave * 16 + lr;
  const int hig = R / p.bq;
  const int rpos = q0 + (R - hig * p.bq);
  const int rh = kvh * p.group + hig;
  const bool rok = hig < p.group && rpos < sq;
  u32x4 qf[KS];
  {
    const uint16_t* qp = p.q + b * p.q_sb + (int64_t)rh * p.q_sh + (qrow0 + rpos) * p.q_ss;
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = rok ? ldg16(qp + s * 32 + lg * 8) : u32x4{0, 0, 0, 0};
  }

  const int pmax = min(q0 + p.bq, sq) - 1;
  const int kv_end = p.causal ? min(L, pmax + off + 1) : L;
  const int n_tiles = kv_end > 0 && q0 < sq ? (kv_end + kPage - 1) / kPage : 0;
  int n_full = L / kPage;
  if (p.causal) n_full = min(n_full, max(q0 + off + 1, 0) / kPage);
  n_full = min(n_full, n_tiles);
  // key tiles [j0, j1) of this workgroup: all of them, or one part of a tail split
  int j0 = 0, j1 = n_tiles;
  if (nsp) {
    const int tp = (n_tiles + nsp - 1) / nsp;
    j0 = min(part * tp, n_tiles);
    j1 = min(n_tiles, j0 + tp);
  }

  const bool paged = p.block_table != nullptr;
  const int64_t rs = paged ? (int64_t)p.hkv * D : p.kv_ss;
  const int r_in = lane / CPR, pc = lane % CPR;
  constexpr int NI2 = 2 * NIW;   // waves 0-3 copy the shares of waves (2w, 2w + 1)
  uint32_t dma_off[NI2];
#pragma unroll
  for (int k = 0; k < NI2; ++k) {
    const int row = ((wave & 3) * NI2 + k) * RPI + r_in;
    dma_off[k] = (uint32_t)((row * rs + ((pc ^ qswz<D>(row)) << 3)) * 2);
  }
  const uint32_t smem_base = lds_addr(smem);
  uint32_t stage_ok = 3u;
  auto issue_tile = [&](int j, int stage) {
    int64_t base;
    bool page_ok = true;
    if (paged) {
      const int pg = scalar_load(p.block_table + (int64_t)b * p.max_blocks + __builtin_amdgcn_readfirstlane(j));
      page_ok = pg >= 0 && pg < p.num_blocks;
      base = (int64_t)(page_ok ? pg : 0) * kPage * p.hkv * D + (int64_t)kvh * D;
    } else {
      base = b * p.kv_sb + kvh * p.kv_sh + (int64_t)j * kPage * p.kv_ss;
    }
    stage_ok = page_ok ? (stage_ok | (1u << stage)) : (stage_ok & ~(1u << stage));
    const uint32_t ks = smem_base + stage * 2 * TILE * 2;
    const uint32_t vs = ks + TILE * 2;
    if (wave >= 4) return;
    if (page_ok && (j + 1) * kPage <= L) {
#pragma unroll
      for (int k = 0; k < NI2; ++k) {
        const int i = wave * NI2 + k;
        dma16_s(p.k + base, dma_off[k], ks + i * 1024);
        dma16_s(p.v + base, dma_off[k], vs + i * 1024);
      }
    } else {
#pragma unroll
      for (int k = 0; k < NI2; ++k) {
        const int i = wave * NI2 + k;
        const bool ok = page_ok && (j * kPage + (i * RPI + r_in) < L);
        dma16_v(ok ? p.k + base + dma_off[k] / 2 : kZeroChunk, ks + i * 1024);
        dma16_v(ok ? p.v + base + dma_off[k] / 2 : kZeroChunk, vs + i * 1024);
      }
    }
  };

  // per-lane LDS read offsets: K rows 16 kb + lr at chunk 4 s + lg (kb as an immediate);
  // V^T reads at row 16 t + 4 lg + lr / 4 (t as an immediate), d 16 db + 4 (lr % 4)
  uint32_t koff[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) koff[s] = lr * ROWB + (((4 * s + lg) ^ qswz<D>(lr)) << 4);
  uint32_t voff[DB];
  {
    const int row = 4 * lg + (lr >> 2);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int chunk = 2 * db + ((lr & 3) >> 1);
      voff[db] = row * ROWB + ((chunk ^ qswz<D>(row)) << 4) + 8 * (lr & 1);
    }
  }

  float mref = -INFINITY, lsum = 0.f;
  float4v acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = float4v{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int j, auto stage_c, auto mask_c) {
    constexpr int STAGE = decltype(stage_c)::value;
    constexpr bool MASK = decltype(mask_c)::value;
    const char* ks = reinterpret_cast<const char*>(smem) + STAGE * 2 * TILE * 2;
    const char* vs = ks + TILE * 2;
    float4v sc[4];   // key block kb: keys 16 kb + 4 lg + i
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) sc[kb] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        sc[kb] = Op<T>::mfma(as_op<T>(*reinterpret_cast<const u32x4*>(ks + koff[s] + kb * 16 * ROWB)),
                             as_op<T>(qf[s]), sc[kb]);
    if constexpr (MASK) {
      // key j * 64 + 16 kb + 4 lg + i is visible iff 16 kb + i < lim (one per-lane bound,
      // compared with constants, so that no per-key value lives across the tile loop)
      const int lim = (p.causal ? min(L, rpos + off + 1) : L) - j * kPage - 4 * lg;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[kb][i] = 16 * kb + i < lim ? sc[kb][i] : -INFINITY;
    }
    float mx = fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                     fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3])));
    mx = fmaxf(mx, fmaxf(fmaxf(fmaxf(sc[2][0], sc[2][1]), fmaxf(sc[2][2], sc[2][3])),
                         fmaxf(fmaxf(sc[3][0], sc[3][1]), fmaxf(sc[3][2], sc[3][3]))));
    // lazily moved reference maximum, as in prefill_kernel; the row spans lanes l, l^16,
    // l^32, l^48
    if (__builtin_amdgcn_ballot_w64(mx * c > mref + kLazy) != 0) {
      const float mt = rows4_max(mx) * c;
      const bool up = mt > mref + kLazy;
      const float nref = up ? mt : mref;
      const float alpha = up ? fast_exp2(mref - nref) : 1.f;
      mref = nref;
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[db] *= alpha;
    }
    const float mneg = mref == -INFINITY ? 0.f : -mref;
    u32x2 pb[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      float y[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) y[i] = fast_exp2(__builtin_fmaf(sc[kb][i], c, mneg));
      pb[kb] = u32x2{pack2<T>(y[0], y[1]), pack2<T>(y[2], y[3])};
    }
    float ps0 = lsum, ps1 = 0.f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      ps0 = Op<T>::sum2(pb[kb][0], ps0);
      ps1 = Op<T>::sum2(pb[kb][1], ps1);
    }
    lsum = ps0 + ps1;
    // O^T += V^T P^T, 32 keys per product: key blocks 2 t2 and 2 t2 + 1, enumerated in the
    // same order in the V^T operand (two transposed reads) and in P (two packed blocks)
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
      const u32x4 pq = u32x4{pb[2 * t2][0], pb[2 * t2][1], pb[2 * t2 + 1][0], pb[2 * t2 + 1][1]};
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const u32x2 lo = lds_read_tr16(reinterpret_cast<const uint16_t*>(vs + voff[db] + 32 * t2 * ROWB));
        const u32x2 hi = lds_read_tr16(reinterpret_cast<const uint16_t*>(vs + voff[db] + (32 * t2 + 16) * ROWB));
        acc[db] = Op<T>::mfma(as_op<T>(u32x4{lo[0], lo[1], hi[0], hi[1]}), as_op<T>(pq), acc[db]);
      }
    }
  };

  using Full = std::integral_constant<bool, false>;
  using Masked = std::integral_constant<bool, true>;
  // step i takes tile j0 + i from stage i % 2
  auto step = [&](int i, auto stage_c, auto mask_c) {
    constexpr int STAGE = decltype(stage_c)::value;
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
    const int j = j0 + i;
    if (j + 1 < j1) issue_tile(j + 1, STAGE ^ 1);
    if ((stage_ok >> STAGE) & 1u) compute(j, stage_c, mask_c);
  };
  // tiles below n_full need no mask, the others do: two loops, so that each loop body
  // holds one kind of tile (one register assignment for the loop-carried state)
  const int h = j1 - j0, nf = max(0, min(n_full, j1) - j0);
  if (h > 0) issue_tile(j0, 0);
  int i = 0;
  for (; i + 1 < nf; i += 2) {
    step(i, std::integral_constant<int, 0>{}, Full{});
    step(i + 1, std::integral_constant<int, 1>{}, Full{});
  }
  if (i < nf) {
    step(i, std::integral_constant<int, 0>{}, Full{});
    ++i;
  }
  // the masked loop is unrolled by two as well: a loop whose body picks one of two stage
  // bodies at run time spills 84 registers here
  if (i < h && (i & 1)) {
    step(i, std::integral_constant<int, 1>{}, Masked{});
    ++i;
  }
  for (; i + 1 < h; i += 2) {
    step(i, std::integral_constant<int, 0>{}, Masked{});
    step(i + 1, std::integral_constant<int, 1>{}, Masked{});
  }
  if (i < h) step(i, std::integral_constant<int, 0>{}, Masked{});

  // ---- epilogue: lane holds d = 16 db + 4 lg + i of its row
  const float l = rows4_sum(lsum);
  if (nsp) {
    // tail split: this part's normalised O and lse in fp32, for the combine; part 0 also
    // records where the row goes (-1 for a padding row)
    const int64_t prow = (int64_t)(lid / nsp) * (16 * NW) + wave * 16 + lr;
    if (rok) {
      const float inv = l > 0.f ? 1.f / l : 0.f;
      float* po = p.part_o + (prow * nsp + part) * D;
#pragma unroll
      for (int db = 0; db < DB; ++db) *reinterpret_cast<float4v*>(po + 16 * db + 4 * lg) = acc[db] * inv;
      if (lg == 0) p.part_lse[prow * nsp + part] = l > 0.f ? (mref + __log2f(l)) * kLn2 : -INFINITY;
    }
    if (lg == 0 && part == 0) {
      p.row_off[prow] = rok ? b * p.o_sb + (int64_t)rh * p.o_sh + (qrow0 + rpos) * p.o_ss : -1;
      p.row_lse[prow] = !(rok && p.lse) ? -1
                        : p.cu_seqlens_q ? (int64_t)rh * scalar_load(p.cu_seqlens_q + p.batch) + qrow0 + rpos
                                         : ((int64_t)b * p.hq + rh) * p.seqlen_q + rpos;
    }
  } else if (rok) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const int64_t ob = b * p.o_sb + (int64_t)rh * p.o_sh + (qrow0 + rpos) * p.o_ss;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int d0 = 16 * db + 4 * lg;
      const float4v v = acc[db] * inv;
      if (p.o_dtype == kF32) {
        *reinterpret_cast<float4v*>(static_cast<float*>(p.o) + ob + d0) = v;
      } else if (p.o_dtype == kF16) {
        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(p.o) + ob + d0) =
            u32x2{pack2<F16>(v[0], v[1]), pack2<F16>(v[2], v[3])};
      } else {
        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(p.o) + ob + d0) =
            u32x2{pack_bf16_round(v[0], v[1], p.o_round), pack_bf16_round(v[2], v[3], p.o_round)};
      }
    }
    if (p.lse && lg == 0) {
      const int64_t li = p.cu_seqlens_q ? (int64_t)rh * scalar_load(p.cu_seqlens_q + p.batch) + qrow0 + rpos
                                        : ((int64_t)b * p.hq + rh) * p.seqlen_q + rpos;
      p.lse[li] = l > 0.f ? (mref + __log2f(l)) * kLn2 : -INFINITY;
    }
  }
}

// Below this many single-group workgroups (four rounds of two per CU on 256 CUs) a causal
// launch splits the key range of each workgroup over two groups (d <= 128): the causal
// triangle then leaves too few long workgroups to balance the CUs. (A non-causal launch
// of that size keeps one group: its workgroups are all equally long, and a one-group
// step is about 10% cheaper.)
constexpr int64_t kSplitBelow = 2048;

template <int D, int NG, int NW, typename T, bool PRECISE, bool PAIR = false>
hipError_t launch_ng(const PrefillParams& p, int64_t blocks, hipStream_t stream) {
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((prefill_kernel<D, NG, NW, T, PRECISE, PAIR>), dim3((unsigned)blocks),
                     dim3(64 * NW * NG), 0, stream, p);
  return hipGetLastError();
}

// Launch form of a prefill: which kernel, its query positions per item and its item count.
struct Form {
  int nw = 4, ng = 1;
  bool pair = false, narrow = false;
  bool fill = false;      // a causal two-group launch that leaves at least half of the CUs idle
  int bq = 0;
  int64_t blocks = 0;     // workgroups of the launch
  int64_t items = 0;      // work items (query blocks of one (sequence, KV head))
};

template <int D, bool PRECISE>
Form choose_form(const PrefillParams& p) {
  Form f;
  if constexpr (D == 128) {
    // Eight-wave workgroups of 256 query rows share each K/V tile. They take every
    // non-causal launch with at least one of them per CU, and every causal launch with at
    // least one and a half per CU (dispatched heaviest first, that many balance the
    // causal triangle; with one per CU the longest item sets the time and the two-group
    // form below is faster).
    // Causal MHA below 8192 keys keeps the four-wave blocks: an eight-wave block of G = 1
    // spans 256 positions, four of its tiles straddle the diagonal, and at these lengths
    // that costs more than the shared copies save (8% at 4096 keys; from 8192 keys on the
    // eight-wave form is ahead).
    // d = 64 keeps four-wave blocks, three workgroups per CU: its tile loop is bound by
    // the softmax, and a third wave per SIMD hides more of it than shared copies save
    // (4.5-11% faster on four d = 64 shapes, causal and not, bit-equal).
    const bool diag_heavy = p.causal && p.group == 1 && p.seqlen_k < 8192;
    const int bq8 = 256 / p.group;
    const int64_t blocks8 = (int64_t)((p.seqlen_q + bq8 - 1) / bq8) * p.hkv * p.batch;
    const int64_t cus = std::max(p.cus, 1);
    if (!diag_heavy && (p.causal ? 2 * blocks8 >= 3 * cus : blocks8 >= cus)) {
      f.nw = 8; f.bq = bq8; f.blocks = f.items = blocks8;
      return f;
    }
  }
  f.bq = 128 / p.group;
  const int64_t nq = (p.seqlen_q + f.bq - 1) / f.bq;
  f.blocks = f.items = nq * p.hkv * p.batch;
  if constexpr (D == 256 && !PRECISE) {
    // d = 256: eight waves of 16 rows (two per SIMD) in place of four of 32 (one per SIMD)
    f.narrow = true; f.nw = 8;
    f.fill = p.causal && 2 * f.blocks <= (int64_t)std::max(p.cus, 1);
    return f;
  }
  if constexpr (D <= 128) {
    if (p.causal && f.blocks < kSplitBelow) {
      // Two-group workgroups fill a CU each. Under a causal mask, pair a heavy and a
      // light query block per workgroup when that still leaves a workgroup per CU.
      f.ng = 2;
      if (nq > 1 && f.blocks >= 2 * (int64_t)std::max(p.cus, 1)) {
        f.pair = true;
        f.blocks = (nq + 1) / 2 * p.hkv * p.batch;
      } else if (2 * f.blocks <= (int64_t)std::max(p.cus, 1)) {
        // few items: their key ranges may instead be split over four-wave workgroups
        // (plan_one decides; launch_one keeps the two-group form if it does not split)
        f.fill = true;
      }
    }
  }
  return f;
}

// Workgroups of a kernel that stay resident on a CU at once (registers and LDS of the
// compiled kernel), asked once per kernel: the one-group form of NW waves, or (NW = 0) the
// narrow d = 256 kernel.
template <int D, int NW, typename T>
hipError_t resident_per_cu(int* n) {
  static std::atomic<int> cached{0};   // the same for every gfx950 device; callers may race
  if (const int c = cached.load(std::memory_order_relaxed); c > 0) {
    *n = c;
    return hipSuccess;
  }
  int v = 0;
  hipError_t e;
  if constexpr (NW == 0) {
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &v, reinterpret_cast<const void*>(&prefill_narrow_kernel<D, T>), 512, 0);
  } else {
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &v, reinterpret_cast<const void*>(&prefill_kernel<D, 1, NW, T, false, false>), 64 * NW, 0);
  }
  if (e != hipSuccess) return e;
  v = std::max(v, 1);
  cached.store(v, std::memory_order_relaxed);
  *n = v;
  return hipSuccess;
}

// Tail split: for launches whose items all have the same key range (non-causal, one
// group); the split pays once the items are long enough that the partial writes and the
// combine cost less than the idle CUs of the last round. The library splits when the
// tail items would leave at least half of the CUs without work: with several resident
// workgroups per CU, a last round that still reaches every CU is not slower in proportion
// to its empty slots (fewer workgroups share each CU), and splitting it did not pay
// (d = 64, a half-full round of three workgroups per CU: +1.6% time).
// Causal launches with few items (their two-group workgroups would leave at least half of
// the CUs idle, as chunked prefill of a few short chunks does) split every item instead,
// over four-wave workgroups, when the keys reach kFillMinTiles tiles: 18-42% faster on
// such shapes, slower with 1024-2048 keys, where the partial writes dominate.
constexpr int kTailMinTiles = 32;     // keys per item >= 2048 when the library chooses
constexpr int kFillMinTiles = 48;     // causal few-item launches: keys >= 3072
constexpr int kTailMaxParts = 16;

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

template <int D, typename T, bool PRECISE>
hipError_t plan_one(const PrefillParams& p, int kv_splits, PrefillPlan* plan) {
  const Form f = choose_form<D, PRECISE>(p);
  *plan = PrefillPlan{};
  plan->items = f.items;
  plan->rows = (f.narrow ? 16 : 32) * f.nw;
  if constexpr (PRECISE) {
    return hipSuccess;
  } else {
    const int n_tiles = (p.seqlen_k + kPage - 1) / kPage;
    const bool fill = f.fill;   // causal few items: every item (one-group or narrow form)
    if (kv_splits == 1 || n_tiles == 0 || !(fill || (!p.causal && f.ng == 1))) return hipSuccess;
    int occ = 1;
    hipError_t e;
    if constexpr (D == 256) e = resident_per_cu<D, 0, T>(&occ);
    else if constexpr (D == 128) e = (f.nw == 8 && !fill) ? resident_per_cu<D, 8, T>(&occ) : resident_per_cu<D, 4, T>(&occ);
    else e = resident_per_cu<D, 4, T>(&occ);
    if (e != hipSuccess) return e;
    const int64_t cap = (int64_t)occ * std::max(p.cus, 1);
    const int64_t tail = fill ? f.items : f.items % cap;
    if (tail == 0) return hipSuccess;
    int64_t parts;
    if (kv_splits >= 2) {
      parts = kv_splits;
    } else if (fill) {
      if (n_tiles < kFillMinTiles) return hipSuccess;
      parts = std::min<int64_t>({std::max<int64_t>(cap / tail, 2), kTailMaxParts, n_tiles / 8});
    } else {
      if (2 * tail > std::max(p.cus, 1) || n_tiles < kTailMinTiles) return hipSuccess;
      parts = std::min<int64_t>({cap / tail, kTailMaxParts, n_tiles / 8});
      if (parts < 2) return hipSuccess;
    }
    const int64_t rows = tail * plan->rows;
    if (tail * parts > 0x7FFFFFFF || rows > 0x7FFFFFFF) return hipSuccess;
    plan->parts = (int32_t)parts;
    plan->tail = tail;
    plan->part_o_off = 0;
    plan->part_lse_off = align256((size_t)rows * parts * D * sizeof(float));
    plan->row_off_off = plan->part_lse_off + align256((size_t)rows * parts * sizeof(float));
    plan->row_lse_off = plan->row_off_off + align256((size_t)rows * sizeof(int64_t));
    plan->bytes = plan->row_lse_off + align256((size_t)rows * sizeof(int64_t));
    return hipSuccess;
  }
}

template <int D, typename T, bool PRECISE>
hipError_t launch_one(const PrefillParams& p0, const PrefillPlan& plan, hipStream_t stream) {
  PrefillParams p = p0;
  const Form f = choose_form<D, PRECISE>(p);
  p.bq = f.bq;
  p.split_parts = 0;
  // one launch of the chosen one-group kernel over `blocks` workgroups
  auto launch1 = [&](const PrefillParams& q, int64_t blocks) -> hipError_t {
    if constexpr (D == 256 && !PRECISE) {
      if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
      hipLaunchKernelGGL((prefill_narrow_kernel<D, T>), dim3((unsigned)blocks), dim3(512), 0, stream, q);
      return hipGetLastError();
    } else {
      if constexpr (D == 128) {
        if (f.nw == 8) return launch_ng<D, 1, 8, T, PRECISE>(q, blocks, stream);
      }
      return launch_ng<D, 1, 4, T, PRECISE>(q, blocks, stream);
    }
  };
  if constexpr (D <= 128) {
    if (f.ng == 2 && !(f.fill && plan.parts >= 2)) {
      return f.pair ? launch_ng<D, 2, 4, T, PRECISE, true>(p, f.blocks, stream)
                    : launch_ng<D, 2, 4, T, PRECISE>(p, f.blocks, stream);
    }
  }
  if (plan.parts < 2) return launch1(p, f.blocks);
  // Tail split: the items before the tail as usual, then (item, part) units of the tail
  // items writing partials, then the log-sum-exp combine of those partials into o.
  const int64_t n_main = f.items - plan.tail;
  if (n_main > 0) {
    if (hipError_t e = launch1(p, n_main); e != hipSuccess) return e;
  }
  PrefillParams q = p;
  q.split_parts = plan.parts;
  q.split_item0 = (int32_t)n_main;
  if (hipError_t e = launch1(q, plan.tail * plan.parts); e != hipSuccess) return e;
  CombineParams c{};
  c.part_o = p.part_o; c.part_lse = p.part_lse; c.o = p.o; c.lse = p.lse;
  c.pairs = (int32_t)(plan.tail * plan.rows); c.num_splits = plan.parts;
  c.o_dtype = p.o_dtype; c.o_round = p.o_round;
  c.row_off = p.row_off; c.row_lse = p.row_lse;
  return launch_combine(c, D, stream);
}

template <int D>
hipError_t plan_d(const PrefillParams& p, int qkv_dtype, bool precise, int kv_splits, PrefillPlan* plan) {
  if (qkv_dtype == kF16)
    return precise ? plan_one<D, F16, true>(p, kv_splits, plan) : plan_one<D, F16, false>(p, kv_splits, plan);
  return precise ? plan_one<D, BF16, true>(p, kv_splits, plan) : plan_one<D, BF16, false>(p, kv_splits, plan);
}

template <int D>
hipError_t launch_d(const PrefillParams& p, const PrefillPlan& plan, int qkv_dtype, bool precise, hipStream_t s) {
  if (qkv_dtype == kF16)
    return precise ? launch_one<D, F16, true>(p, plan, s) : launch_one<D, F16, false>(p, plan, s);
  return precise ? launch_one<D, BF16, true>(p, plan, s) : launch_one<D, BF16, false>(p, plan, s);
}

}  // namespace

hipError_t plan_prefill(const PrefillParams& p, int head_dim, int qkv_dtype, bool precise, int kv_splits,
                        PrefillPlan* plan) {
  switch (head_dim) {
    case 64: return plan_d<64>(p, qkv_dtype, precise, kv_splits, plan);
    case 128: return plan_d<128>(p, qkv_dtype, precise, kv_splits, plan);
    case 256: return plan_d<256>(p, qkv_dtype, precise, kv_splits, plan);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_prefill(const PrefillParams& p, const PrefillPlan& plan, int head_dim, int qkv_dtype,
                          bool precise, hipStream_t stream) {
  switch (head_dim) {
    case 64: return launch_d<64>(p, plan, qkv_dtype, precise, stream);
    case 128: return launch_d<128>(p, plan, qkv_dtype, precise, stream);
    case 256: return launch_d<256>(p, plan, qkv_dtype, precise, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace attn
