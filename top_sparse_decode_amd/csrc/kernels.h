// kernels.h -- internal kernel argument blocks and launchers (not part of
// the public ABI; see include/sparse_decode.h for that).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sd {

struct ScoreArgs {
  const int32_t* block_table;
  const int32_t* kv_lens;
  int32_t batch, max_pages, max_kv_len;
  const void* k;
  int32_t dtype;  // 0 f32, 1 bf16 (q has the same type); 2 fp8 e4m3 codes (q bf16)
  const float* k_scale;  // fp8: row scales [num_pages][num_kv_heads][page_size]
  int32_t num_pages, page_size, num_kv_heads, head_dim;
  int64_t page_stride, head_stride, token_stride;
  const void* q;
  int32_t q_heads;
  const float* head_weights;
  int32_t mode;  // 0 group sum, 1 group mean, 2 relu weighted
  float head_scale;
  float inv_g;
  float* scores;     // [batch][num_kv_heads][max_kv_len]
  float* row_bound;  // [batch][num_kv_heads] or null
  int32_t* row_stats;  // selection statistics (min/max keys of finite scores) or null
  // fused path (fast scorers): each block writes (kmin key, kmax key, bound
  // bits, 0) to span_slots[row][blockIdx.x] instead of the row_stats / row_bound
  // atomics, and clears its share of the row's row_stats (so no separate
  // initialisation pass is needed)
  int32_t* span_slots;
};

// Per-row selection statistics: [kmin key, kmax key, band count, cut (4
// slots), score floor certified by the hint (float bits, -inf = none),
// 2048-bin histogram, arrival counters of the one-launch selection's two row
// barriers, 6 unused].  Cleared by the fast scorer or select_init.
constexpr int kStatStride = 8 + 2048 + 8;
constexpr int kStatBarrier = 8 + 2048;
constexpr int kSelChunk = 4096;   // tokens per block in the multi-block selection
constexpr int kBandCap = 4096;    // band entries kept per row before falling back

struct SelectArgs {
  const float* scores;  // [batch][groups][row_stride]
  int32_t batch, groups, row_stride;
  const int32_t* kv_lens;
  int32_t k;
  int32_t* indices;     // [batch][groups][k]
  int32_t* counts;      // [batch][groups] or null
  float* keys;          // scratch, same shape as scores
  float* row_bound;     // fast scores: per-row bound on |fast - exact| (zeroed by init); null = exact
  ScoreArgs score;      // fast scores: the inputs needed to re-score band tokens exactly
  int32_t* stats;       // [rows][kStatStride]
  int32_t* chunk_counts;  // [rows][nchunks][2]: kept-for-sure count, -inf count
  uint64_t* band;       // [rows][kBandCap]: (key << 32) | ~position
  int32_t nchunks;      // ceil(row_stride / kSelChunk)
  // optional hint: a previous selection per row (request-local positions),
  // used only to certify a lower score floor for the histogram range
  const int32_t* hint;  // [rows][hint_stride] or null
  int32_t hint_len;
  int64_t hint_stride;
  // optional copy of this selection (the next step's hint), written by emit
  int32_t* writeback;   // [rows][wb_stride] or null
  int64_t wb_stride;
  // fast scores from the fused path: the scorer's per-block slots; the
  // histogram pass reduces them into stats[0..1] and row_bound
  const int32_t* span_slots;  // [rows][nspans][4] or null
  int32_t nspans;
  // one-launch selection: how long a block waits at a row barrier before it
  // finishes its row alone (wall-clock ticks, 100 MHz; 0 = the default)
  int64_t spin_ticks;
};

struct AttnArgs {
  const int32_t* block_table;
  const int32_t* kv_lens;
  int32_t batch, max_pages, max_kv_len;
  const void* q;
  int32_t q_heads;
  int32_t dtype;  // q, k, v share it
  const void* k;
  int32_t k_num_pages, page_size, num_kv_heads, head_dim;
  int64_t k_page_stride, k_head_stride, k_token_stride;
  const void* v;
  int32_t v_num_pages;
  int64_t v_page_stride, v_head_stride, v_token_stride;
  int32_t v_dim;
  const int32_t* indices;  // [batch][num_kv_heads][k_sel]
  int32_t k_sel;
  float scale;
  int32_t splits, chunk;  // split s covers index slots [s*chunk, (s+1)*chunk)
  float* part_o;          // [batch][q_heads][splits][v_dim]
  float* part_ml;         // [batch][q_heads][splits][2]
  void* out;
  int32_t out_dtype;
};

// TriAttention normalize + reduce (tri.hip)
struct TriArgs {
  const float* scores;     // [layers][batch][groups][row_stride]
  int32_t layers, batch, groups, row_stride;
  const int32_t* kv_lens;  // [batch]
  int32_t mode;            // 0 per layer per head, 1 per head, 2 union
  double* stats;           // [layers*batch*groups][4]: mu, sigma, RN(1 / sigma), (unused)
  int32_t* lens;           // [layers*batch]: kv_lens repeated per layer (mode 0), or null
  float* reduced;          // [out_rows][row_stride]
  int32_t exact_slow;      // 1: every sum by long accumulation (set by launch_tri)
  int32_t z_rows;          // 1: the statistics kernel writes each member's z row (set by launch_tri)
  int32_t want_reduced;    // 1: the caller reads the reduced rows
  // per layer and head, with tri_fuses_select(): the statistics kernel also
  // selects each member row's k largest z (indices [members][k], counts)
  int32_t sel_k;
  int32_t* sel_indices;
  int32_t* sel_counts;
};
bool tri_fuses_select(const TriArgs& a);
int tri_out_rows(int layers, int batch, int groups, int mode);
hipError_t launch_tri(const TriArgs& a, hipStream_t st);

bool score_exact_supported(int G);
bool score_fast_supported(const ScoreArgs& a);
hipError_t launch_score_exact(const ScoreArgs& a, hipStream_t st);
hipError_t launch_score_fast(const ScoreArgs& a, hipStream_t st);
// blocks per row of the fast scorer's grid, and an upper bound for any device
int score_fast_spans(const ScoreArgs& a);
int score_fast_max_spans(int max_kv_len);

int select_max_row();
size_t select_workspace_bytes(int rows, int row_stride);
void select_bind_workspace(SelectArgs* a, void* ws);
// init must run before the scorer (or launch_select_stats) writes row_stats
hipError_t launch_select_init(const SelectArgs& a, hipStream_t st);
hipError_t launch_select_stats(const SelectArgs& a, hipStream_t st);
hipError_t launch_select(const SelectArgs& a, hipStream_t st);
// exact scores, rows up to 16384 tokens: the whole selection in one launch
// (needs neither init nor statistics; hints are not used)
bool select_short_path(const SelectArgs& a);
hipError_t launch_select_short(const SelectArgs& a, hipStream_t st);

bool attn_mla_supported(const AttnArgs& a);
bool attn_vec_supported(const AttnArgs& a);
int attn_rows_per_split(const AttnArgs& a, bool mla);
hipError_t launch_attn(const AttnArgs& a, hipStream_t st);

hipError_t launch_fill_f32(float* p, int64_t n, float v, hipStream_t st);
// block-granular selections: entry e of a row -> tokens e*bs .. e*bs+bs-1 below kv_len, else -1
hipError_t launch_expand_blocks(const int32_t* blocks, const int32_t* kv_lens, int32_t batch, int32_t groups,
                                int32_t k_blocks, int32_t block_size, int32_t cap, int32_t* tok, hipStream_t st);
// multi-query decode: row b*n + j <- block-table row b, kv_len max(kv_lens[b] - (n - 1 - j), 0)
hipError_t launch_mq_expand(const int32_t* bt, const int32_t* kv_lens, int32_t batch, int32_t max_pages,
                            int32_t n, int32_t* bt_out, int32_t* kv_out, hipStream_t st);
hipError_t launch_local_to_global(const int32_t* bt, int32_t max_pages, int32_t batch,
                                  int32_t page_size, int32_t num_pages, const int32_t* local,
                                  int32_t groups, int32_t k, int64_t* out, hipStream_t st);

}  // namespace sd
