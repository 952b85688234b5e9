// Internal interface of the latent sparse attention kernel (msa_latent.hip)
// for the host API (msa_api.cpp).
#pragma once

#include "msa_kernels.h"

namespace msa {

// One leaf of the latent cache: its pool and how sequences map into it.
struct LatentLeaf {
  Pool pool;
  const int32_t* clen;    // [B] entries (window leaf: positions) cached
  const int32_t* table;   // [B][stride] page ids
  int32_t stride;
};

struct LatentParams {
  const uint16_t* q;      // bf16 [R][H][128]
  const int32_t* offs;    // [B+1]
  int32_t batch, max_seq;
  const int32_t* lists;   // [R][H_lat][top_c] compressed-leaf entries
  int32_t top_c;
  const float* sink;      // [H]
  LatentLeaf swa, comp;
  int32_t fp8;            // 1: the leaves this launch reads are FP8 e4m3 (scale-free), 0: BF16
  int32_t H, H_lat, G;    // query heads, latent heads, query heads per latent head
  int32_t ncg;            // column groups of 64 query heads per latent head
  int32_t window, np, rcap;  // np: partitions of this launch
  int32_t pi_base;        // index of this launch's first partition among the row's
  int32_t np_total;       // partitions of the row over every launch of the call
  float scale_log2;       // softmax scale * log2(e)
  uint16_t* out;          // bf16 [R][H][128]
  float* part_o;          // [np][rcap][H][128]
  float* part_lse;        // [np][rcap][H]
  uint64_t* ready;        // split-K ready flags [group][np] (msa_splitk.h)
  uint64_t epoch;         // per call, never 0
  uint32_t* err;          // device error word (bad table data), or null
};

// Most list slots (entries) one partition of a latent row may hold.
constexpr int kLatentMaxSlots = 2048;
// Entries per latent tile.
constexpr int kLatentTile = 32;

hipError_t launch_latent(const LatentParams& p, hipStream_t s);

}  // namespace msa
