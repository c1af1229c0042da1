// Kernel parameter blocks and launchers (internal to libattn.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// Debug builds (compiled with -DATTN_POISON_LDS=1, as libattn_poison.so) fill each
// kernel's LDS with NaN bit patterns before its first use, so that a read of LDS that no
// copy or store wrote reaches the output as NaN. Release builds compile none of it.
#ifndef ATTN_POISON_LDS
#define ATTN_POISON_LDS 0
#endif

namespace attn {

constexpr bool kPoisonLds = ATTN_POISON_LDS != 0;

enum DType { kF16 = 0, kBF16 = 1, kF32 = 2 };

struct PrefillParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  void* o;
  float* lse;
  const int32_t* block_table;   // null for dense K/V
  const int32_t* seqlens_k;     // null: every sequence has seqlen_k keys
  const int32_t* cu_seqlens_q;  // null, or [B + 1] first packed query row of each sequence
  int64_t q_sb, q_sh, q_ss;     // element strides of Q over (batch, head, position)
  int64_t o_sb, o_sh, o_ss;     // same for O (elements of o_dtype)
  int64_t kv_sb, kv_sh, kv_ss;  // dense K/V strides over (batch, kv head, position)
  int32_t batch, hq, hkv, group, seqlen_q, seqlen_k;
  int32_t num_blocks, max_blocks;
  int32_t bq;                   // query positions per workgroup (rows = group * bq <= 128)
  int32_t causal, o_dtype;
  int32_t o_round;              // rounding of a bf16 output: 0 RTNE, 1 RTNA, 2 RTZ
  float scale_log2;             // softmax scale * log2(e)
  int32_t cus;                  // compute units of the device (work pairing decision)
  // Tail split (non-causal launches whose last round of work items would leave CUs idle):
  // a second launch gives each of the last items' key tiles to split_parts workgroups,
  // which write fp32 partials that the combine merges. split_parts = 0 in ordinary
  // launches. In a split launch, workgroup unit u takes part u % split_parts of item
  // split_item0 + u / split_parts.
  int32_t split_parts, split_item0;
  float* part_o;                // [tail rows, split_parts, d]: O of each part, normalised
  float* part_lse;              // [tail rows, split_parts]: natural-log lse of each part
  int64_t* row_off;             // [tail rows]: element offset of the row in o, -1 if no row
  int64_t* row_lse;             // [tail rows]: index of the row in lse, -1 if none
};

// What a prefill launch does with a given shape on the current device (host side).
struct PrefillPlan {
  int64_t items;                // work items of the chosen launch form
  int32_t rows;                 // query rows per item (32 per wave)
  int32_t parts;                // key parts per tail item (0: no tail split)
  int64_t tail;                 // items split (the last `tail` items)
  size_t part_o_off, part_lse_off, row_off_off, row_lse_off, bytes;   // workspace layout
};

struct DecodeParams {
  const uint16_t* q;            // [B, Hq, d]
  const uint16_t* k;            // [num_blocks, 64, Hkv, d]
  const uint16_t* v;
  const int32_t* block_table;   // [B, max_blocks]
  const int32_t* seqlens_k;     // [B]
  float* part_o;                // [B, Hq, num_splits, d]
  float* part_lse;              // [B, Hq, num_splits]
  int32_t batch, hq, hkv, group;
  int32_t num_blocks, max_blocks, max_seqlen_k, num_splits;
  int32_t part_tokens;          // keys per split (multiple of 64), partition kernel only
  float scale_log2;
  // balanced (stream) kernel: plan written by the plan kernel into the workspace
  int32_t* plan;                // {total units per KV head, units per workgroup, workgroups used}
  int32_t* prefix;              // [B + 1] first unit of each sequence's run
  int32_t* start;               // [nwk] run holding the first unit of each workgroup range
  int32_t nwk;                  // workgroups launched per KV head
};

struct CombineParams {
  const float* part_o;          // [B*H, S, d]
  const float* part_lse;        // [B*H, S]
  void* o;                      // [B*H, d]
  float* lse;                   // optional [B*H]
  const int32_t* seqlens_k;     // optional [B]: sequences with no key give O = 0, lse = -inf
  int32_t heads;                // H (to find the sequence of a (b, h) pair)
  int32_t max_seqlen_k;
  int32_t pairs, num_splits, o_dtype;
  int32_t o_round;              // rounding of a bf16 output: 0 RTNE, 1 RTNA, 2 RTZ
  // optional row map (prefill tail splits): pair i goes to element offset row_off[i] of o
  // (skipped when negative) and to lse[row_lse[i]] (none when negative)
  const int64_t* row_off;
  const int64_t* row_lse;
};

// Launch form and tail split of a prefill launch (kv_splits: 0 = chosen by the library,
// 1 = never split, n >= 2 = split the tail items into n parts). Returns hipSuccess or the
// error of the occupancy query.
hipError_t plan_prefill(const PrefillParams& p, int head_dim, int qkv_dtype, bool precise, int kv_splits,
                        PrefillPlan* plan);
// Each launcher returns hipSuccess or the launch error; shapes were validated by the caller.
// With plan.parts >= 2, p.part_o, p.part_lse, p.row_off and p.row_lse point into a
// workspace laid out as the plan says.
hipError_t launch_prefill(const PrefillParams& p, const PrefillPlan& plan, int head_dim, int qkv_dtype,
                          bool precise, hipStream_t stream);
hipError_t launch_decode_split(const DecodeParams& p, int head_dim, int qkv_dtype,
                               hipStream_t stream);
// Plan kernel then the balanced split kernel (num_splits >= 2); grid = nwk * hkv.
hipError_t launch_decode_stream(const DecodeParams& p, int head_dim, int qkv_dtype,
                                hipStream_t stream);
hipError_t launch_combine(const CombineParams& p, int head_dim, hipStream_t stream);

}  // namespace attn
