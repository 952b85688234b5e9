// Host side of libmsa: argument validation, route choice, split-K sizing,
// workspace carving and kernel launches on the caller's stream.
//
// Routes follow the "msa" page of the MAX Mojo docs (routes paragraph): the
// maximum number of new tokens of any sequence picks the kernels -- 1 is a
// decode step, 2..8 a speculative-decode step, more a prefill step -- and
// every route takes the same arguments.  Grid sizes derive from host bounds
// only, never from device data, so launches are graph-capturable.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdint>
#include <cstring>

#include "msa.h"
#include "msa_kernels.h"
#include "msa_latent.h"

namespace {

using namespace msa;

static_assert(kErrPage == MSA_DEVERR_PAGE && kErrLength == MSA_DEVERR_LENGTH,
              "device error bits match the header");

constexpr size_t kAlign = 256;
constexpr int kMaxPartitions = 64;
constexpr int kMaxDevices = 64;
constexpr size_t kMaxLds = 64 * 1024;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Per-device facts read once: compute-unit count and whether it is gfx950.
std::atomic<int> g_dev_cus[kMaxDevices];
std::atomic<int> g_dev_ok[kMaxDevices];   // 0 unknown, 1 gfx950, -1 other

int current_device(int* cus) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MSA_ERR_DEVICE;
  int ok = g_dev_ok[dev].load();
  if (ok == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MSA_ERR_DEVICE;
    ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    g_dev_cus[dev].store(prop.multiProcessorCount);
    g_dev_ok[dev].store(ok);
  }
  if (ok != 1) return MSA_ERR_DEVICE;
  if (cus) *cus = g_dev_cus[dev].load();
  return MSA_OK;
}

enum class Route { Decode, Spec, Prefill };

Route route_of(const msa_ragged& rg) {
  if (rg.max_seq_length <= 1) return Route::Decode;
  if (rg.max_seq_length <= MSA_MAX_SPEC_DRAFT) return Route::Spec;
  return Route::Prefill;
}

// Blocks the longest possible sequence may hold.
int64_t max_blocks(const msa_ragged& rg) {
  return ((int64_t)rg.max_cache_length + rg.max_seq_length + MSA_BLOCK_SIZE - 1) / MSA_BLOCK_SIZE;
}

// Blocks the kernels may address per sequence: the host bound, and never
// past the sequence's row of the lookup table, so that lengths beyond the
// table (bad device data) cannot move a table read into the next row or
// past the table.
int32_t block_bound(const msa_ragged& rg) {
  return (int32_t)std::min<int64_t>(max_blocks(rg), rg.lookup_stride);
}

int64_t row_capacity(const msa_ragged& rg) { return (int64_t)rg.batch * rg.max_seq_length; }

int check_ragged(const msa_ragged* rg) {
  if (!rg) return MSA_ERR_NULL;
  if (rg->batch < 0 || rg->max_seq_length < 0 || rg->max_cache_length < 0) return MSA_ERR_PARAM;
  if (rg->batch == 0 || rg->max_seq_length == 0) return MSA_OK;
  if (!rg->input_row_offsets || !rg->cache_lengths || !rg->kv_lookup_table) return MSA_ERR_NULL;
  if (rg->lookup_stride < 1) return MSA_ERR_SHAPE;
  if (max_blocks(*rg) > MSA_MAX_BLOCKS) return MSA_ERR_SHAPE;
  if (row_capacity(*rg) > (int64_t)INT32_MAX / 8) return MSA_ERR_SHAPE;
  return MSA_OK;
}

bool empty_batch(const msa_ragged& rg) { return rg.batch == 0 || rg.max_seq_length == 0; }

enum class CacheRole { IndexK, KV };

int check_cache(const msa_paged_cache* c, CacheRole role) {
  if (!c) return MSA_ERR_NULL;
  if (!c->data) return MSA_ERR_NULL;
  if (c->dtype != MSA_DTYPE_BF16 && c->dtype != MSA_DTYPE_FP8_E4M3) return MSA_ERR_DTYPE;
  if (c->page_size != MSA_BLOCK_SIZE || c->head_dim != MSA_HEAD_DIM) return MSA_ERR_SHAPE;
  if (c->num_pages < 1 || c->num_heads < 1) return MSA_ERR_SHAPE;
  const int64_t esz = c->dtype == MSA_DTYPE_BF16 ? 2 : 1;
  if (reinterpret_cast<uintptr_t>(c->data) % 16) return MSA_ERR_SHAPE;
  for (int64_t st : {c->page_stride, c->head_stride, c->token_stride})
    if (st < 0 || (st * esz) % 16) return MSA_ERR_SHAPE;
  if (c->token_stride < MSA_HEAD_DIM) return MSA_ERR_SHAPE;
  // kernels address the rows of one page with 32-bit byte offsets
  if (c->token_stride * esz * MSA_BLOCK_SIZE > (int64_t)INT32_MAX) return MSA_ERR_SHAPE;
  // per-token scales: exactly the FP8 index-K cache has them
  const bool scaled = role == CacheRole::IndexK && c->dtype == MSA_DTYPE_FP8_E4M3;
  if (!scaled && c->scale) return MSA_ERR_DTYPE;
  if (scaled) {
    if (!c->scale) return MSA_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(c->scale) % 16) return MSA_ERR_SHAPE;
    for (int64_t st : {c->scale_page_stride, c->scale_head_stride})
      if (st < 0 || st % 4) return MSA_ERR_SHAPE;
  }
  return MSA_OK;
}

Pool pool_of(const msa_paged_cache& c) {
  return Pool{c.data, c.page_stride, c.head_stride, c.token_stride, c.num_pages,
              c.scale, c.scale_page_stride, c.scale_head_stride};
}

Ragged ragged_of(const msa_ragged& rg) {
  return Ragged{rg.input_row_offsets, rg.cache_lengths, rg.kv_lookup_table, rg.lookup_stride,
                rg.batch, rg.max_seq_length};
}

int check_selection(int32_t top_k, int32_t init_blocks, int32_t local_blocks) {
  if (top_k < 1 || top_k > MSA_MAX_TOPK) return MSA_ERR_PARAM;
  if (init_blocks < 0 || local_blocks < 0) return MSA_ERR_PARAM;
  if ((int64_t)init_blocks + local_blocks > top_k) return MSA_ERR_PARAM;
  return MSA_OK;
}

bool aligned16(const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; }

// ---- indexer ---------------------------------------------------------------

// Prefill indexer tiles: the index-K head count is only known with the
// cache; the work list is sized for the worst case (one head per KV head).
size_t indexer_items(const msa_ragged& rg, int32_t num_kv_heads, int32_t H_ik) {
  const int tq = prefill_indexer_tile(num_kv_heads, H_ik);
  return (size_t)rg.batch * ((rg.max_seq_length + tq - 1) / tq) * H_ik;
}

size_t indexer_ws(const msa_ragged& rg, int32_t num_kv_heads, int32_t top_k) {
  if (empty_batch(rg)) return 0;
  const int64_t nb = max_blocks(rg);
  if (nb <= top_k) return 0;     // every row selects all of its blocks
  const size_t stride = (size_t)(nb + 15) / 16 * 16;
  size_t ws = align_up((size_t)row_capacity(rg) * num_kv_heads * stride * sizeof(float));
  if (route_of(rg) == Route::Prefill)
    ws += align_up(2 * sizeof(int32_t)) +
          align_up(std::max(indexer_items(rg, num_kv_heads, 1), indexer_items(rg, num_kv_heads, num_kv_heads)) *
                   sizeof(int32_t));
  return ws;
}

// ---- attention ---------------------------------------------------------------

struct AttnPlan {
  int tpw, ntg, np, tgs;
};

// Tokens per wave and waves (token groups) per workgroup of the decode
// kernel, and the workgroups of token groups per (sequence, KV head).
void decode_tiling(const msa_ragged& rg, int G, int* tpw, int* ntg, int* ntgb) {
  const Route r = route_of(rg);
  *tpw = r == Route::Decode ? 1 : std::min(16 / G, std::max(1, rg.max_seq_length));
  if (r == Route::Prefill) *tpw = 16 / G;
  const int ntok_groups = (rg.max_seq_length + *tpw - 1) / *tpw;
  *ntg = std::min(4, ntok_groups);
  *ntgb = (ntok_groups + *ntg - 1) / *ntg;
}

// Speculative rows of two to four token groups, in one partition: one wave
// per workgroup instead of one workgroup per (sequence, KV head).  A
// workgroup of four token groups puts every wave of a sequence with many
// draft tokens on one CU, and a CU streams at most about 43 GB/s however
// many of its waves are busy; one-wave workgroups, the busy token groups
// first, spread the busy waves over the CUs.  The waves still walk their
// unions on one common schedule, each computing it from every token group's
// selections.
void one_wave_groups(Route r, int ntok_groups, AttnPlan* pl) {
  pl->tgs = 1;
  if (r == Route::Spec && pl->tpw > 1 && ntok_groups >= 2 && ntok_groups <= 4 && pl->np == 1) {
    pl->ntg = 1;
    pl->tgs = ntok_groups;
  }
}

AttnPlan plan_attention(const msa_ragged& rg, int G, int H_kv, int top_k, int req_np, int cus) {
  AttnPlan pl{};
  const Route r = route_of(rg);
  int ntgb = 0;
  decode_tiling(rg, G, &pl.tpw, &pl.ntg, &ntgb);
  const int ntok_groups = (rg.max_seq_length + pl.tpw - 1) / pl.tpw;
  pl.tgs = 1;
  if (r == Route::Prefill) {
    pl.np = 1;
    return pl;
  }
  if (req_np > 0) {
    pl.np = req_np;
    one_wave_groups(r, ntok_groups, &pl);
    return pl;
  }
  // CU fill.  Measured on the decode workloads: once the batch alone gives
  // two streaming waves per CU, one partition is fastest (no partial writes,
  // no merge); below that, split until about three waves per CU (the FP8
  // 128k decode: 6 partitions 0.585 of HBM peak against 0.56 with 8 and
  // 0.51 with 4), but keep at least two blocks per partition when the batch
  // already gives a few waves per CU.
  const int64_t base = (int64_t)rg.batch * H_kv * ntok_groups;
  int64_t np = 1;
  if (base < (int64_t)cus * 2) {
    const int64_t target = (int64_t)cus * 3;
    np = (target + base - 1) / std::max<int64_t>(1, base);
    const int union_blocks = std::min<int64_t>(top_k * pl.tpw, max_blocks(rg));
    const int min_per = base >= cus / 2 ? 2 : 1;
    np = std::min<int64_t>(np, std::max(1, union_blocks / min_per));
  }
  pl.np = (int)std::max<int64_t>(1, std::min<int64_t>(np, kMaxPartitions));
  one_wave_groups(r, ntok_groups, &pl);
  return pl;
}

// Union-tile plan slots for `waves` waves per workgroup: tokens per tile
// for group size G and KV type (the kernels' choice).  Workspace is sized
// for the smaller tile of the two types, since the size query does not know
// the type.
size_t prefill_plan_slots(const msa_ragged& rg, int G, int H_kv, int waves) {
  int tq_b = 0, tq_f = 0, nct = 0;
  prefill_tiling(G, false, waves, &tq_b, &nct);
  prefill_tiling(G, true, waves, &tq_f, &nct);
  const int tq = std::min(tq_b, tq_f);
  return (size_t)rg.batch * ((rg.max_seq_length + tq - 1) / tq) * H_kv;
}

// Dense-causal slots of the prefill route get their own kernel (8 waves of
// two MFMA column tiles, whose K and V^T operand reads each feed two MFMAs)
// at group sizes where that kernel's tiles have the union-tile kernel's
// token count.  Measured on the dense-causal sequences of the prefill
// workload (BF16 KV): 0.39 against 0.37 of MFMA peak.  On sparse tiles
// the same kernel loses (a wave's four tokens choose more blocks between
// them: 0.155 against 0.170), so those keep the 16-wave kernel.
bool dense_split(int G) { return G == 8 || G == 16; }

// Workspace of the union-tile route: plan counts, ids, pages, masks, the
// work list and the scheduler state (and, on the prefill route, a second
// work list and scheduler state for the dense-causal slots).
size_t union_ws(const msa_ragged& rg, int H_q, int H_kv, int waves) {
  const size_t slots = prefill_plan_slots(rg, H_q / H_kv, H_kv, waves);
  const size_t nb = (size_t)max_blocks(rg);
  const size_t lists = waves == kUnionWavesPrefill && dense_split(H_q / H_kv) ? 2 : 1;
  return align_up(slots * sizeof(int32_t)) +
         lists * (align_up(slots * sizeof(int32_t)) + align_up(kSchedInts * sizeof(int32_t))) +
         3 * align_up(slots * nb * sizeof(int32_t));
}

// Split-K workspace of the decode kernel: the ready flags (one per
// partition of each workgroup of token groups of a (sequence, KV head)),
// then the partial outputs and log-sum-exps of every partition.
size_t splitk_counters(const msa_ragged& rg, int G, int H_kv) {
  int tpw = 0, ntg = 0, ntgb = 0;
  decode_tiling(rg, G, &tpw, &ntg, &ntgb);
  return (size_t)rg.batch * H_kv * ntgb;
}

size_t splitk_ws(const msa_ragged& rg, int H_q, int H_kv, int np) {
  const size_t rows = (size_t)np * row_capacity(rg) * H_q;
  return align_up(splitk_counters(rg, H_q / H_kv, H_kv) * np * sizeof(uint64_t)) +
         align_up(rows * MSA_HEAD_DIM * sizeof(float)) + align_up(rows * sizeof(float));
}

// Epoch stamped into a call's split-K ready flags: never 0, new per call.
std::atomic<uint64_t> g_epoch{0};
uint64_t next_epoch() {
  for (;;) {
    const uint64_t e = g_epoch.fetch_add(1) + 1;
    if (e) return e;
  }
}

// Workspace one call needs: the union-tile route (prefill, and speculative
// rows under msa_attention_paged_shared) or split-K partials.
size_t attention_ws(const msa_ragged& rg, int H_q, int H_kv, int np, bool shared) {
  if (empty_batch(rg)) return 0;
  if (route_of(rg) == Route::Prefill) return union_ws(rg, H_q, H_kv, kUnionWavesPrefill);
  if (shared && route_of(rg) == Route::Spec) return union_ws(rg, H_q, H_kv, kUnionWavesShared);
  if (np <= 1) return 0;
  return splitk_ws(rg, H_q, H_kv, np);
}

int check_heads(int32_t num_q_heads, int32_t num_kv_heads) {
  if (num_kv_heads < 1 || num_kv_heads > MSA_MAX_KV_HEADS || num_q_heads < num_kv_heads ||
      num_q_heads % num_kv_heads)
    return MSA_ERR_SHAPE;
  const int G = num_q_heads / num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16) return MSA_ERR_SHAPE;
  return MSA_OK;
}

// ---- latent attention ------------------------------------------------------------

// Column groups of 64 query heads per latent head.
int latent_col_groups(int G) { return (G + 63) / 64; }

int64_t latent_max_tiles(int32_t window, int32_t top_c) {
  return ((int64_t)window + top_c + kLatentTile - 1) / kLatentTile;
}

int check_latent_shape(int32_t batch, int32_t max_seq_length, int32_t num_heads,
                       int32_t num_latent_heads, int32_t window, int32_t top_c, int32_t num_partitions) {
  if (batch < 0 || max_seq_length < 0) return MSA_ERR_PARAM;
  if (num_latent_heads < 1 || num_heads < num_latent_heads || num_heads % num_latent_heads)
    return MSA_ERR_SHAPE;
  if (window < 0 || window > MSA_LATENT_MAX_WINDOW) return MSA_ERR_PARAM;
  if (top_c < 0 || top_c > MSA_LATENT_MAX_TOPC) return MSA_ERR_PARAM;
  if (num_partitions < 0 || num_partitions > kMaxPartitions) return MSA_ERR_PARAM;
  if ((int64_t)batch * max_seq_length > (int64_t)INT32_MAX / 8) return MSA_ERR_SHAPE;
  return MSA_OK;
}

// Partitions: enough that one partition's entries fit the kernel's LDS list;
// when automatic, enough workgroups for one per CU (the kernel's LDS holds
// one workgroup per CU), with at least two tiles per partition.
int plan_latent(int32_t batch, int32_t max_seq_length, int32_t num_heads, int32_t num_latent_heads,
                int32_t window, int32_t top_c, int32_t req, int cus) {
  const int64_t tiles = std::max<int64_t>(1, latent_max_tiles(window, top_c));
  const int64_t per_max = kLatentMaxSlots / kLatentTile;
  const int64_t min_np = (tiles + per_max - 1) / per_max;
  if (req > 0) return req >= min_np ? req : MSA_ERR_PARAM;
  const int64_t base = (int64_t)batch * max_seq_length * num_latent_heads *
                       latent_col_groups(num_heads / num_latent_heads);
  int64_t np = ((int64_t)cus + base - 1) / std::max<int64_t>(1, base);
  np = std::min<int64_t>(np, std::max<int64_t>(1, tiles / 2));
  np = std::max(np, min_np);
  return (int)std::min<int64_t>(np, kMaxPartitions);
}

// Leaves of two storage types: the window leaf's tiles and the list's go
// through two launches (one tile format each) as disjoint partition sets of
// one split-K, np_swa partitions for the window positions and np_comp for
// the list slots, in proportion to their tiles, each at least one and
// enough that a partition's entries fit the kernel's LDS list.
void latent_split(int32_t window, int32_t top_c, int np, int* np_swa, int* np_comp) {
  const int64_t ta = std::max<int64_t>(1, ((int64_t)window + kLatentTile - 1) / kLatentTile);
  const int64_t tb = std::max<int64_t>(1, ((int64_t)top_c + kLatentTile - 1) / kLatentTile);
  const int64_t per_max = kLatentMaxSlots / kLatentTile;
  const int64_t need_a = (ta + per_max - 1) / per_max, need_b = (tb + per_max - 1) / per_max;
  const int64_t total = std::max<int64_t>(std::max<int64_t>(np, 2), need_a + need_b);
  int64_t a = (total * ta + (ta + tb) / 2) / (ta + tb);
  a = std::max(need_a, std::min(a, total - need_b));
  *np_swa = (int)a;
  *np_comp = (int)(total - a);
}

// Partitions of a call: both leaves read -> the two-type split's total
// (also what the size query reserves, since it does not know the types).
int latent_total_partitions(int32_t window, int32_t top_c, int np) {
  if (window <= 0 || top_c <= 0) return np;
  int a = 0, b = 0;
  latent_split(window, top_c, np, &a, &b);
  return std::max(np, a + b);
}

// Split-K workspace of the latent kernel: ready flags (one per partition of
// each (row slot, latent head, column group)), partial outputs and
// log-sum-exps.
size_t latent_groups(int32_t batch, int32_t max_seq_length, int32_t num_heads,
                     int32_t num_latent_heads) {
  return (size_t)batch * max_seq_length * num_latent_heads *
         latent_col_groups(num_heads / num_latent_heads);
}

size_t latent_ws(int32_t batch, int32_t max_seq_length, int32_t num_heads,
                 int32_t num_latent_heads, int np) {
  if (np <= 1 || batch == 0 || max_seq_length == 0) return 0;
  const size_t rows = (size_t)np * batch * max_seq_length * num_heads;
  return align_up(latent_groups(batch, max_seq_length, num_heads, num_latent_heads) * np *
                  sizeof(uint64_t)) +
         align_up(rows * MSA_HEAD_DIM * sizeof(float)) + align_up(rows * sizeof(float));
}

int check_latent_leaf(const msa_latent_leaf* lf, int32_t num_latent_heads, int64_t need_entries) {
  if (!lf) return MSA_ERR_NULL;
  int st = check_cache(&lf->cache, CacheRole::KV);
  if (st != MSA_OK) return st;
  if (lf->cache.num_heads != num_latent_heads) return MSA_ERR_SHAPE;
  // kernels pack (page, slot) into 32 bits
  if (lf->cache.num_pages > (1 << 24)) return MSA_ERR_SHAPE;
  if (!lf->cache_lengths || !lf->lookup_table) return MSA_ERR_NULL;
  if (lf->max_cache_length < 0) return MSA_ERR_PARAM;
  if (lf->lookup_stride < 1 || (int64_t)lf->lookup_stride * MSA_BLOCK_SIZE < need_entries) return MSA_ERR_SHAPE;
  return MSA_OK;
}

LatentLeaf leaf_of(const msa_latent_leaf* lf) {
  return LatentLeaf{pool_of(lf->cache), lf->cache_lengths, lf->lookup_table, lf->lookup_stride};
}

}  // namespace

extern "C" {

const char* msa_status_string(int status) {
  switch (status) {
    case MSA_OK: return "ok";
    case MSA_ERR_NULL: return "null pointer";
    case MSA_ERR_SHAPE: return "unsupported shape, stride or alignment";
    case MSA_ERR_PARAM: return "parameter out of range";
    case MSA_ERR_DTYPE: return "unsupported storage type";
    case MSA_ERR_WORKSPACE: return "workspace too small";
    case MSA_ERR_LAUNCH: return "kernel launch failed";
    case MSA_ERR_DEVICE: return "no gfx950 device";
    case MSA_ERR_SCRATCH: return "shape needs more workspace than the fixed scratch array holds";
    default: return "unknown status";
  }
}

size_t msa_indexer_workspace_bytes(const msa_ragged* rg, int32_t num_kv_heads, int32_t top_k) {
  if (check_ragged(rg) != MSA_OK || num_kv_heads < 1 || num_kv_heads > MSA_MAX_KV_HEADS ||
      top_k < 1)
    return 0;
  return indexer_ws(*rg, num_kv_heads, top_k);
}

int msa_indexer_paged(int32_t* d_indices, const void* q_idx, const msa_paged_cache* index_k,
                      const msa_ragged* rg, int32_t num_kv_heads, int32_t top_k,
                      int32_t init_blocks, int32_t local_blocks, void* workspace,
                      size_t workspace_bytes, void* stream) {
  int st = check_ragged(rg);
  if (st != MSA_OK) return st;
  if ((st = check_selection(top_k, init_blocks, local_blocks)) != MSA_OK) return st;
  // the prefill scorer's tile holds 256 (token, KV head) columns of one
  // index-K head, so at most 256 KV heads may share it
  if (num_kv_heads < 1 || num_kv_heads > MSA_MAX_KV_HEADS) return MSA_ERR_SHAPE;
  if (empty_batch(*rg)) return MSA_OK;   // no rows: buffers may be empty (null)
  if ((st = check_cache(index_k, CacheRole::IndexK)) != MSA_OK) return st;
  if (index_k->num_heads != 1 && index_k->num_heads != num_kv_heads) return MSA_ERR_SHAPE;
  if (!d_indices || !q_idx) return MSA_ERR_NULL;
  if (!aligned16(q_idx) || !aligned16(d_indices)) return MSA_ERR_SHAPE;
  const size_t need = indexer_ws(*rg, num_kv_heads, top_k);
  if (need && !workspace) return MSA_ERR_NULL;
  if (workspace_bytes < need) return MSA_ERR_WORKSPACE;
  if ((st = current_device(nullptr)) != MSA_OK) return st;

  IndexerParams p{};
  p.q_idx = static_cast<const uint16_t*>(q_idx);
  p.ik = pool_of(*index_k);
  p.ik_fp8 = index_k->dtype == MSA_DTYPE_FP8_E4M3;
  p.rg = ragged_of(*rg);
  p.scores = static_cast<float*>(workspace);
  p.d_indices = d_indices;
  p.nbmax = block_bound(*rg);
  p.score_stride = (p.nbmax + 15) / 16 * 16;
  p.H_kv = num_kv_heads;
  p.H_ik = index_k->num_heads;
  p.top_k = top_k;
  p.init = init_blocks;
  p.local = local_blocks;
  p.err = device_error_word();
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (p.nbmax > top_k) {
    hipError_t e;
    int cus = 0;
    if ((st = current_device(&cus)) != MSA_OK) return st;
    if (route_of(*rg) == Route::Prefill) {
      p.tq = prefill_indexer_tile(num_kv_heads, p.H_ik);
      p.ntiles = (rg->max_seq_length + p.tq - 1) / p.tq;
      const size_t stride = (size_t)p.score_stride;
      char* w = static_cast<char*>(workspace) +
                align_up((size_t)row_capacity(*rg) * num_kv_heads * stride * sizeof(float));
      p.sched = reinterpret_cast<int32_t*>(w);
      p.worklist = reinterpret_cast<int32_t*>(w + align_up(2 * sizeof(int32_t)));
      e = launch_indexer_prefill(p, cus, s);
    } else {
      e = launch_indexer_decode(p, cus, s);
    }
    if (e != hipSuccess) return MSA_ERR_LAUNCH;
  }
  if (launch_topk(p, s) != hipSuccess) return MSA_ERR_LAUNCH;
  return MSA_OK;
}

int msa_indexer_reuse(int32_t* d_indices, const int32_t* prev_indices, const int32_t* src_row,
                      int32_t rows, int32_t prev_rows, int32_t num_kv_heads, int32_t top_k,
                      void* stream) {
  if (rows < 0 || prev_rows < 0 || num_kv_heads < 1) return MSA_ERR_PARAM;
  if (top_k < 1 || top_k > MSA_MAX_TOPK) return MSA_ERR_PARAM;
  if (rows == 0) return MSA_OK;
  if (!d_indices || !prev_indices || !src_row) return MSA_ERR_NULL;
  if ((int64_t)rows * num_kv_heads * top_k > (int64_t)INT32_MAX ||
      (int64_t)prev_rows * num_kv_heads * top_k > (int64_t)INT32_MAX)
    return MSA_ERR_SHAPE;
  const int st = current_device(nullptr);
  if (st != MSA_OK) return st;
  if (launch_indexer_reuse(d_indices, prev_indices, src_row, rows, prev_rows,
                           num_kv_heads * top_k, static_cast<hipStream_t>(stream)) != hipSuccess)
    return MSA_ERR_LAUNCH;
  return MSA_OK;
}

int msa_latent_partitions(int32_t batch, int32_t max_seq_length, int32_t num_heads,
                          int32_t num_latent_heads, int32_t window, int32_t top_c,
                          int32_t num_partitions) {
  int st = check_latent_shape(batch, max_seq_length, num_heads, num_latent_heads, window, top_c,
                              num_partitions);
  if (st != MSA_OK) return st;
  int cus = 256;
  if (num_partitions == 0 && current_device(&cus) != MSA_OK) cus = 256;
  return plan_latent(batch, max_seq_length, num_heads, num_latent_heads, window, top_c,
                     num_partitions, cus);
}

size_t msa_latent_workspace_bytes(int32_t batch, int32_t max_seq_length, int32_t num_heads,
                                  int32_t num_latent_heads, int32_t window, int32_t top_c,
                                  int32_t num_partitions) {
  const int np = msa_latent_partitions(batch, max_seq_length, num_heads, num_latent_heads, window,
                                       top_c, num_partitions);
  if (np < 1) return 0;
  return latent_ws(batch, max_seq_length, num_heads, num_latent_heads,
                   latent_total_partitions(window, top_c, np));
}

int msa_latent_attention_paged(void* output, const void* q, const int32_t* input_row_offsets,
                               int32_t batch, int32_t max_seq_length, const int32_t* comp_indices,
                               int32_t top_c, const float* attn_sink, const msa_latent_leaf* swa,
                               const msa_latent_leaf* comp, int32_t num_heads,
                               int32_t num_latent_heads, int32_t window, float scale,
                               int32_t num_partitions, void* workspace, size_t workspace_bytes,
                               void* stream) {
  int st = check_latent_shape(batch, max_seq_length, num_heads, num_latent_heads, window, top_c,
                              num_partitions);
  if (st != MSA_OK) return st;
  if (!(scale > 0.f) || scale > 3.0e38f) return MSA_ERR_PARAM;   // positive and finite
  if (batch == 0 || max_seq_length == 0) return MSA_OK;
  if (!output || !q || !input_row_offsets || !attn_sink) return MSA_ERR_NULL;
  if (!aligned16(output) || !aligned16(q)) return MSA_ERR_SHAPE;
  if (window > 0) {
    if (!swa) return MSA_ERR_NULL;
    if ((st = check_latent_leaf(swa, num_latent_heads,
                                (int64_t)swa->max_cache_length + max_seq_length)) != MSA_OK)
      return st;
  }
  if (top_c > 0) {
    if (!comp || !comp_indices) return MSA_ERR_NULL;
    if ((st = check_latent_leaf(comp, num_latent_heads, comp->max_cache_length)) != MSA_OK) return st;
  }
  // Leaves of one storage type take one launch; leaves of two types take
  // one launch per leaf (one tile format each) as disjoint partition sets
  // of one split-K, merged by the list launch's last partition.
  const bool mixed = window > 0 && top_c > 0 && comp->cache.dtype != swa->cache.dtype;
  const int leaf_dtype = window > 0 ? swa->cache.dtype
                         : top_c > 0 ? comp->cache.dtype
                                     : (int)MSA_DTYPE_BF16;
  int cus = 0;
  if (num_partitions == 0 && (st = current_device(&cus)) != MSA_OK) return st;
  const int np = plan_latent(batch, max_seq_length, num_heads, num_latent_heads, window, top_c,
                             num_partitions, cus);
  if (np < 1) return np;
  int np_swa = 0, np_comp = 0;
  if (mixed) latent_split(window, top_c, np, &np_swa, &np_comp);
  const int np_total = mixed ? np_swa + np_comp : np;
  const size_t need = latent_ws(batch, max_seq_length, num_heads, num_latent_heads, np_total);
  if (need && !workspace) return MSA_ERR_NULL;
  if (workspace_bytes < need) return MSA_ERR_WORKSPACE;
  const int ncg = latent_col_groups(num_heads / num_latent_heads);
  if ((int64_t)batch * max_seq_length * num_latent_heads * ncg * np_total > (int64_t)INT32_MAX)
    return MSA_ERR_SHAPE;
  if (num_partitions != 0 && (st = current_device(&cus)) != MSA_OK) return st;

  LatentParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.offs = input_row_offsets;
  p.batch = batch;
  p.max_seq = max_seq_length;
  p.lists = comp_indices;
  p.top_c = top_c;
  p.sink = attn_sink;
  if (window > 0) p.swa = leaf_of(swa);
  if (top_c > 0) p.comp = leaf_of(comp);
  p.fp8 = leaf_dtype == MSA_DTYPE_FP8_E4M3;
  p.H = num_heads;
  p.H_lat = num_latent_heads;
  p.G = num_heads / num_latent_heads;
  p.ncg = ncg;
  p.window = window;
  p.np = np;
  p.pi_base = 0;
  p.np_total = np_total;
  p.rcap = batch * max_seq_length;
  p.scale_log2 = scale * 1.4426950408889634f;  // log2(e)
  p.out = static_cast<uint16_t*>(output);
  p.err = device_error_word();
  if (np_total > 1) {
    // flags, partial outputs, partial log-sum-exps; the kernel's last
    // partition of each group merges (no separate combine launch)
    const size_t rows = (size_t)np_total * p.rcap * num_heads;
    char* w = static_cast<char*>(workspace);
    p.ready = reinterpret_cast<uint64_t*>(w);
    w += align_up(latent_groups(batch, max_seq_length, num_heads, num_latent_heads) * np_total *
                  sizeof(uint64_t));
    p.part_o = reinterpret_cast<float*>(w);
    w += align_up(rows * MSA_HEAD_DIM * sizeof(float));
    p.part_lse = reinterpret_cast<float*>(w);
    p.epoch = next_epoch();
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!mixed) {
    if (launch_latent(p, s) != hipSuccess) return MSA_ERR_LAUNCH;
    return MSA_OK;
  }
  // the window leaf's partitions (the row's first ones, holding the sink) ...
  LatentParams a = p;
  a.top_c = 0;
  a.np = np_swa;
  a.fp8 = swa->cache.dtype == MSA_DTYPE_FP8_E4M3;
  if (launch_latent(a, s) != hipSuccess) return MSA_ERR_LAUNCH;
  // ... then the list's, whose last partition merges all of them
  LatentParams c = p;
  c.window = 0;
  c.np = np_comp;
  c.pi_base = np_swa;
  c.fp8 = comp->cache.dtype == MSA_DTYPE_FP8_E4M3;
  if (launch_latent(c, s) != hipSuccess) return MSA_ERR_LAUNCH;
  return MSA_OK;
}

int msa_attention_partitions(const msa_ragged* rg, int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t top_k, int32_t num_partitions) {
  int st = check_ragged(rg);
  if (st != MSA_OK) return st;
  if ((st = check_heads(num_q_heads, num_kv_heads)) != MSA_OK) return st;
  if (top_k < 1 || top_k > MSA_MAX_TOPK) return MSA_ERR_PARAM;
  if (num_partitions < 0 || num_partitions > kMaxPartitions) return MSA_ERR_PARAM;
  if (empty_batch(*rg)) return 1;
  int cus = 256;
  if (num_partitions == 0 && current_device(&cus) != MSA_OK) cus = 256;
  return plan_attention(*rg, num_q_heads / num_kv_heads, num_kv_heads, top_k, num_partitions, cus).np;
}

size_t msa_attention_workspace_bytes(const msa_ragged* rg, int32_t num_q_heads,
                                     int32_t num_kv_heads, int32_t top_k, int32_t num_partitions) {
  const int np = msa_attention_partitions(rg, num_q_heads, num_kv_heads, top_k, num_partitions);
  if (np < 1) return 0;
  // Enough for either entry point: split-K partials, or the union-tile plan
  // that msa_attention_paged_shared builds for speculative rows.
  return std::max(attention_ws(*rg, num_q_heads, num_kv_heads, np, false),
                  attention_ws(*rg, num_q_heads, num_kv_heads, np, true));
}

}  // extern "C"

namespace msa {

// All attention entry points.  `shared` sends speculative rows through the
// union-tile kernel (four waves per workgroup) instead of split-K decode.
int attention_paged_entry(void* output, const void* q, const int32_t* d_indices,
                    const msa_paged_cache* k_cache, const msa_paged_cache* v_cache,
                    const msa_ragged* rg, int32_t num_q_heads, int32_t num_kv_heads, int32_t top_k,
                    float scale, int32_t num_partitions, void* workspace, size_t workspace_bytes,
                    void* stream, bool shared) {
  int st = check_ragged(rg);
  if (st != MSA_OK) return st;
  if ((st = check_heads(num_q_heads, num_kv_heads)) != MSA_OK) return st;
  if (top_k < 1 || top_k > MSA_MAX_TOPK) return MSA_ERR_PARAM;
  if (num_partitions < 0 || num_partitions > kMaxPartitions) return MSA_ERR_PARAM;
  if (!(scale > 0.f) || scale > 3.0e38f) return MSA_ERR_PARAM;   // positive and finite
  if (empty_batch(*rg)) return MSA_OK;   // no rows: buffers may be empty (null)
  if ((st = check_cache(k_cache, CacheRole::KV)) != MSA_OK) return st;
  if ((st = check_cache(v_cache, CacheRole::KV)) != MSA_OK) return st;
  if (k_cache->dtype != v_cache->dtype) return MSA_ERR_DTYPE;
  if (k_cache->num_heads != num_kv_heads || v_cache->num_heads != num_kv_heads) return MSA_ERR_SHAPE;
  if (k_cache->num_pages != v_cache->num_pages) return MSA_ERR_SHAPE;
  if (!output || !q || !d_indices) return MSA_ERR_NULL;
  if (!aligned16(output) || !aligned16(q) || !aligned16(d_indices)) return MSA_ERR_SHAPE;
  // The automatic partition count depends on the device's CU count; an
  // explicit one does not, so its workspace is checked before any device query.
  int cus = 0;
  if (num_partitions == 0 && (st = current_device(&cus)) != MSA_OK) return st;
  const int G = num_q_heads / num_kv_heads;
  const Route route = route_of(*rg);
  const bool union_tiles = route == Route::Prefill || (shared && route == Route::Spec);
  AttnPlan pl = plan_attention(*rg, G, num_kv_heads, top_k, num_partitions, cus);
  if (union_tiles) pl.np = 1;
  const size_t need = attention_ws(*rg, num_q_heads, num_kv_heads, pl.np, shared);
  if (need && !workspace) return MSA_ERR_NULL;
  if (workspace_bytes < need) return MSA_ERR_WORKSPACE;
  if (num_partitions != 0 && (st = current_device(&cus)) != MSA_OK) return st;

  AttnParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.d_indices = d_indices;
  p.k = pool_of(*k_cache);
  p.v = pool_of(*v_cache);
  p.rg = ragged_of(*rg);
  p.H_q = num_q_heads;
  p.H_kv = num_kv_heads;
  p.G = G;
  p.top_k = top_k;
  p.tpw = pl.tpw;
  p.ntg = pl.ntg;
  p.tgs = pl.tgs;
  p.np = pl.np;
  p.rcap = (int32_t)row_capacity(*rg);
  p.nbmax = block_bound(*rg);
  p.scale_log2 = scale * 1.4426950408889634f;  // log2(e)
  p.out = static_cast<uint16_t*>(output);
  p.err = device_error_word();
  const bool fp8 = k_cache->dtype == MSA_DTYPE_FP8_E4M3;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (union_tiles) {
    const int waves = route == Route::Prefill ? kUnionWavesPrefill : kUnionWavesShared;
    // Speculative rows (one tile per sequence and KV head, slots of similar
    // size): each workgroup builds its slot's plan, with no plan or schedule
    // launch.  The prefill route's many uneven slots keep the heaviest-first
    // work list.
    p.inline_plan = waves == kUnionWavesShared ? 1 : 0;
    int nct = 0;
    prefill_tiling(G, fp8, waves, &p.tq, &nct);
    p.ntiles = (rg->max_seq_length + p.tq - 1) / p.tq;
    const size_t slots = prefill_plan_slots(*rg, G, num_kv_heads, waves);
    char* w = static_cast<char*>(workspace);
    p.plan_cnt = reinterpret_cast<int32_t*>(w);
    w += align_up(slots * sizeof(int32_t));
    p.plan_ids = reinterpret_cast<int32_t*>(w);
    w += align_up(slots * (size_t)p.nbmax * sizeof(int32_t));
    p.plan_pages = reinterpret_cast<int32_t*>(w);
    w += align_up(slots * (size_t)p.nbmax * sizeof(int32_t));
    p.plan_mask = reinterpret_cast<uint32_t*>(w);
    w += align_up(slots * (size_t)p.nbmax * sizeof(int32_t));
    p.worklist = reinterpret_cast<int32_t*>(w);
    w += align_up(slots * sizeof(int32_t));
    p.sched = reinterpret_cast<int32_t*>(w);
    w += align_up(kSchedInts * sizeof(int32_t));
    p.dense_list = nullptr;
    p.dense_sched = nullptr;
    if (waves == kUnionWavesPrefill && dense_split(G)) {
      p.dense_list = reinterpret_cast<int32_t*>(w);
      w += align_up(slots * sizeof(int32_t));
      p.dense_sched = reinterpret_cast<int32_t*>(w);
    }
    p.nwg = cus;   // one 142 KiB workgroup per CU
    if ((size_t)(p.nbmax + 1) * sizeof(uint32_t) > kMaxLds) return MSA_ERR_SHAPE;
    if (launch_attention_prefill(p, fp8, waves, s) != hipSuccess) return MSA_ERR_LAUNCH;
    return MSA_OK;
  }
  if (pl.np > 1) {
    // counters, partial outputs, partial log-sum-exps; the kernel's last
    // partition of each group merges (no separate combine launch)
    const size_t rows = (size_t)pl.np * p.rcap * num_q_heads;
    char* w = static_cast<char*>(workspace);
    p.ready = reinterpret_cast<uint64_t*>(w);
    w += align_up(splitk_counters(*rg, G, num_kv_heads) * pl.np * sizeof(uint64_t));
    p.part_o = reinterpret_cast<float*>(w);
    w += align_up(rows * MSA_HEAD_DIM * sizeof(float));
    p.part_lse = reinterpret_cast<float*>(w);
    p.epoch = next_epoch();
  }
  if (attention_decode_lds_bytes(p) > kMaxLds) return MSA_ERR_PARAM;
  if (launch_attention_decode(p, fp8, s) != hipSuccess) return MSA_ERR_LAUNCH;
  return MSA_OK;
}

}  // namespace msa

extern "C" {

int msa_attention_paged(void* output, const void* q, const int32_t* d_indices,
                        const msa_paged_cache* k_cache, const msa_paged_cache* v_cache,
                        const msa_ragged* rg, int32_t num_q_heads, int32_t num_kv_heads,
                        int32_t top_k, float scale, int32_t num_partitions, void* workspace,
                        size_t workspace_bytes, void* stream) {
  return msa::attention_paged_entry(output, q, d_indices, k_cache, v_cache, rg, num_q_heads,
                                    num_kv_heads, top_k, scale, num_partitions, workspace,
                                    workspace_bytes, stream, false);
}

int msa_attention_paged_shared(void* output, const void* q, const int32_t* d_indices,
                               const msa_paged_cache* k_cache, const msa_paged_cache* v_cache,
                               const msa_ragged* rg, int32_t num_q_heads, int32_t num_kv_heads,
                               int32_t top_k, float scale, int32_t num_partitions, void* workspace,
                               size_t workspace_bytes, void* stream) {
  return msa::attention_paged_entry(output, q, d_indices, k_cache, v_cache, rg, num_q_heads,
                                    num_kv_heads, top_k, scale, num_partitions, workspace,
                                    workspace_bytes, stream, true);
}

int msa_splitk_combine(void* output, const float* partial_o, const float* partial_lse,
                       const int32_t* input_row_offsets, int32_t batch, int32_t max_seq_length,
                       int32_t num_partitions, int32_t num_q_heads, void* stream) {
  if (batch < 0 || max_seq_length < 0 || num_partitions < 1 || num_partitions > kMaxPartitions ||
      num_q_heads < 1)
    return MSA_ERR_PARAM;
  if (batch == 0 || max_seq_length == 0) return MSA_OK;
  if (!output || !partial_o || !partial_lse || !input_row_offsets) return MSA_ERR_NULL;
  if (!aligned16(output) || !aligned16(partial_o)) return MSA_ERR_SHAPE;
  if ((int64_t)batch * max_seq_length > (int64_t)INT32_MAX / 8) return MSA_ERR_SHAPE;
  const int st = current_device(nullptr);
  if (st != MSA_OK) return st;
  CombineParams c{partial_o, partial_lse, input_row_offsets, static_cast<uint16_t*>(output), batch,
                  max_seq_length, num_partitions, num_q_heads, batch * max_seq_length};
  if (launch_combine(c, static_cast<hipStream_t>(stream)) != hipSuccess) return MSA_ERR_LAUNCH;
  return MSA_OK;
}

}  // extern "C"
