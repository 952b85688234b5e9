// Internal interface between the host API (msa_api.cpp) and the kernel
// translation units.  Parameter blocks are passed to kernels by value.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

struct msa_paged_cache;
struct msa_ragged;

namespace msa {

// Bits of the per-device error word (the values of msa.h's MSA_DEVERR_*):
// bad table data that a kernel met, skipped or clipped.
constexpr uint32_t kErrPage = 1u;     // a page id outside the pool
constexpr uint32_t kErrLength = 2u;   // a length beyond the host bounds or the table

// A paged cache as the kernels see it: base pointer and element strides,
// plus the per-token scales of an FP8 index-K cache (null otherwise).
struct Pool {
  const void* data;
  int64_t page_stride, head_stride, token_stride;  // elements
  int32_t num_pages;
  const float* scale;                               // [page][head][128 slots]
  int64_t scale_page_stride, scale_head_stride;     // floats
};

// The ragged batch.
struct Ragged {
  const int32_t* offs;    // [B+1]
  const int32_t* clen;    // [B]
  const int32_t* table;   // [B][stride]
  int32_t stride;
  int32_t batch;
  int32_t max_seq;
};

struct IndexerParams {
  const uint16_t* q_idx;  // bf16 [R][H_kv][128]
  Pool ik;                // H_ik heads: bf16, or fp8 e4m3 codes + per-token scales
  int32_t ik_fp8;         // 1: FP8 index-K
  Ragged rg;
  float* scores;          // [rcap][H_kv][score_stride]
  int32_t* d_indices;     // [R][H_kv][top_k]
  int32_t nbmax;
  int32_t score_stride;   // nbmax rounded up to 16
  // prefill route: tiles of tq tokens, scheduled through a device work list
  int32_t tq, ntiles;     // tokens per tile, tiles per sequence
  int32_t* worklist;      // [B * ntiles * H_ik] tile items, heaviest first
  int32_t* sched;         // [0] items in the list, [1] next item to take
  int32_t H_kv, H_ik;
  int32_t top_k, init, local;
  uint32_t* err;          // device error word (bad table data), or null
};

struct AttnParams {
  const uint16_t* q;      // bf16 [R][H_q][128]
  const int32_t* d_indices;
  Pool k, v;
  Ragged rg;
  int32_t H_q, H_kv, G, top_k;
  int32_t tpw;            // tokens per wave (decode / speculative route)
  int32_t ntg;            // token groups (waves) per workgroup
  // token groups of one (sequence, KV head) that one-wave workgroups
  // schedule together (speculative rows, one partition); 1 otherwise
  int32_t tgs;
  int32_t np;             // split-K partitions
  int32_t rcap;           // rows of the partial buffers (batch * max_seq)
  int32_t nbmax;          // blocks a sequence may hold (bitmap size)
  float scale_log2;       // softmax scale * log2(e)
  uint16_t* out;          // bf16 [R][H_q][128]
  float* part_o;          // [np][rcap][H_q][128]
  float* part_lse;        // [np][rcap][H_q]
  // split-K ready flags, [group of token groups of a (sequence, KV head)][np]:
  // a partition stores the call's epoch when its partial is complete; the
  // merging partition (np - 1) clears them
  uint64_t* ready;
  uint64_t epoch;         // per call, never 0
  // prefill route: tiles of tq tokens and the device-built plan
  int32_t tq, ntiles;     // tokens per tile, tiles per sequence
  // union-tile kernel: one workgroup per slot that builds the slot's plan
  // itself (no plan and schedule launches), or persistent workgroups over
  // the work list
  int32_t inline_plan;
  int32_t* plan_cnt;      // [B][ntiles][H_kv] union size
  int32_t* plan_ids;      // [B][ntiles][H_kv][nbmax] ascending block ids
  int32_t* plan_pages;    // [B][ntiles][H_kv][nbmax] page id of each block
  uint32_t* plan_mask;    // [B][ntiles][H_kv][nbmax] token mask per block
  int32_t* worklist;      // [B * ntiles * H_kv] non-empty plan slots, one list per XCD
  int32_t* sched;         // kSchedInts: per XCD list, its length, next entry and start
  // dense-causal tiles (every token chose every block it sees): a second
  // work list for the dense-tile kernel, or null when every slot goes to the
  // list above
  int32_t* dense_list;
  int32_t* dense_sched;
  int32_t nwg;            // persistent workgroups launched
  uint32_t* err;          // device error word (bad table data), or null
};

struct CombineParams {
  const float* part_o;
  const float* part_lse;
  const int32_t* offs;
  uint16_t* out;
  int32_t batch, max_seq, np, H_q, rcap;
};

// Launchers; each returns hipSuccess or the launch error.
hipError_t launch_indexer_decode(const IndexerParams& p, int num_cus, hipStream_t s);
// out[r][:] = prev[src[r]][:] (row length `width` ints), -1 rows for sources
// outside [0, prev_rows)
hipError_t launch_indexer_reuse(int32_t* out, const int32_t* prev, const int32_t* src, int rows,
                                int prev_rows, int width, hipStream_t s);
hipError_t launch_indexer_prefill(const IndexerParams& p, int num_cus, hipStream_t s);
int prefill_indexer_tile(int H_kv, int H_ik);
hipError_t launch_topk(const IndexerParams& p, hipStream_t s);
hipError_t launch_attention_decode(const AttnParams& p, bool fp8, hipStream_t s);
hipError_t launch_combine(const CombineParams& p, hipStream_t s);
// Ints of the union-tile route's scheduler state (three per XCD list).
constexpr int kSchedInts = 24;
// Waves of the union-tile attention kernel per workgroup: the prefill route,
// and speculative rows whose sequences share one selection.
constexpr int kUnionWavesPrefill = 16;
constexpr int kUnionWavesDense = 8;     // dense-causal tiles: 8 waves x 32 columns
constexpr int32_t kPlanDense = 1 << 30; // plan_cnt flag of a dense-causal slot
constexpr int kUnionWavesShared = 4;
hipError_t launch_attention_prefill(const AttnParams& p, bool fp8, int waves, hipStream_t s);

// Tokens per tile (tq) and MFMA column tiles per wave of the union-tile
// attention for group size G, KV storage type and waves per workgroup.
void prefill_tiling(int G, bool fp8, int waves, int* tq, int* nct);

// Bytes of LDS the decode attention kernel needs per workgroup.
size_t attention_decode_lds_bytes(const AttnParams& p);

// Device address of the current device's error word (msa_errors.hip), or
// null if it cannot be resolved.
uint32_t* device_error_word();

// The body of the attention entry points (validation, plan, launches) with
// the workspace given; `shared` picks the union-tile kernel for speculative
// rows (msa_attention_paged_shared).
int attention_paged_entry(void* output, const void* q, const int32_t* d_indices,
                          const msa_paged_cache* k_cache, const msa_paged_cache* v_cache,
                          const msa_ragged* rg, int32_t num_q_heads, int32_t num_kv_heads,
                          int32_t top_k, float scale, int32_t num_partitions, void* workspace,
                          size_t workspace_bytes, void* stream, bool shared);

}  // namespace msa
