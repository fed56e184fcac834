// Launch interface between the C ABI (api.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mdm {

struct Geometry {
  int B, H, Hkv, D, V, seq_len, R;
  int slots;        // cache slots per (sequence, kv head), multiple of kKeyTile
  int table_rows;   // V + 1 + R
  int max_pos;      // seq_len + R
  int hidden;       // H * D
  bool fp32;        // MDM_FP32 storage
};

// Rows [0, n_a): token tok[b*stride + r] (or the mask token V when tok == NULL),
// position pos[b*stride + r] (or r when pos == NULL).  Rows [n_a, n_a + n_reg):
// register r - n_a (id V+1+j, position seq_len+j).  Writes keys (RoPE'd) when
// kc != NULL and transposed values when vc != NULL to slots slot0 + r; records
// (pos, id) when cache_pos != NULL.  When qout != NULL the same launch also writes the rows'
// RoPE'd queries for all H heads: qout[b][h][q_rows][d], row r at index r.
struct AppendArgs {
  const void* tk;
  const void* tv;
  void* kc;
  void* vc;
  int32_t* cache_pos;
  int32_t* cache_tok;
  const float* rope_cos;
  const float* rope_sin;
  const int32_t* tok;
  const int32_t* pos;
  int64_t stride;           // of tok (and of pos when pos_stride is 0)
  int64_t pos_stride;
  int n_a, n_reg, slot0;
  int* err;
  const void* tq;           // query table (with qout)
  void* qout;               // bf16 [B][H][q_rows][d] or NULL
  int q_rows;
};
hipError_t launch_append(const Geometry& g, const AppendArgs& a, hipStream_t s);

// Value tables of the transient keys (bf16): mvt[kvh][d][0..7] = value of the
// mask token, rvt[kvh][d][j] = value of register j (0 for j >= R).
hipError_t launch_value_tables(const Geometry& g, const void* tv, void* mvt, void* rvt, int r_pad, hipStream_t s);

// bf16 attention: C keys staged in LDS per block (bounds max_decode), and the
// key-split partial-result slots (one per block of a split launch).
constexpr int kAttnMaxDecode = 2048;
constexpr int kAttnSplitBlocks = 256;   // split only while fewer blocks than this
constexpr int kAttnMaxSplit = 8;
constexpr int kAttnMinSplitTiles = 6;   // key tiles per block at least (fewer: the combine pass costs more than the split saves)

struct AttnArgs {
  const void* tq;
  const void* tv;           // value table (fp32 path: transient C and R values)
  const void* ktab;         // [H_kv][ktab_rows][d] keys of the mask token at every
                            // position, then of the registers (built at init)
  int ktab_rows;
  const void* mvt;          // bf16 [H_kv][d][8]: the mask token's value, 8 copies
  const void* rvt;          // bf16 [H_kv][d][r_pad]: register values, zero past R
  int r_pad;                // R rounded up to the key tile
  const void* qtab;         // bf16 [H][qtab_rows][d]: RoPE'd queries of the mask token at
                            // every position, then of the registers (built at init)
  int qtab_rows;
  const void* qbuf;         // bf16 [B][H][qbuf_rows][d]: RoPE'd queries of the D rows written
                            // by the preceding append, or NULL (then RoPE in the kernel)
  int qbuf_rows;
  float* part_o;            // [kAttnSplitBlocks][8 waves][32 rows][d] split partial O
  float* part_ml;           // [kAttnSplitBlocks][8 waves][32 rows][2] (reference, row sum)
  const void* kc;
  const void* vc;
  const float* rope_cos;
  const float* rope_sin;
  const int32_t* d_tok;
  const int32_t* d_pos;
  int64_t d_stride;
  const int32_t* c_pos;
  int64_t c_stride;
  float* out;
  int* err;
  int n_d, n_c, n_r;   // query rows: D | C | R
  int S;               // cache length including D
  // Upper-layer (transient) mode, bf16 only: queries of every row from qbuf;
  // the keys/values of the C|R rows from tk [B][H_kv][t_pad][d] and
  // tvt [B][H_kv][d][t_pad] (the launcher passes them as one segment of
  // n_c + n_r keys after the cache).
  const void* tk;
  const void* tvt;
  int t_pad;
  // Optional bf16 copies of the C rows' outputs for the logits, row m = b*n_c + c
  // of [B*n_c][hidden]: pack_hi = the output rounded to bf16, pack_lo = the
  // remainder rounded to bf16 (or NULL).  The same rounding as k_pack.
  uint16_t* pack_hi;
  uint16_t* pack_lo;
};
hipError_t launch_attention(const Geometry& g, const AttnArgs& a, hipStream_t s);

struct VocabArgs {
  const void* w;            // [V][hidden] elem
  // Optional tiled copy of a bf16 W for the wide screen's operand stream (or
  // NULL): wt[rt][c][h][r][e] = W[128 rt + r][64 c + 32 h + e], zero past V,
  // for rt < align_up(V, 512) / 128, so a 128-row x 32-column piece of a
  // stage is one contiguous 8 KB run.  Every other reader uses w.
  const uint16_t* wt;
  const float* h;           // fp32 rows: row m = (b, c) at h + b*h_stride + c*hidden
  int64_t h_stride;
  int n_c;                  // rows per sequence
  uint16_t* hhi;            // [m_pad][hidden] bf16 workspace (bf16 mode)
  uint16_t* hlo;            // [m_pad][hidden] bf16 workspace (accurate mode), or NULL
  float* partials;          // [m_pad][ceil(V / 128)][8]: one record per 128-column tile
  float* zpart;             // split partial logits [n_split][M][v_pad] (bf16 path)
  int64_t zpart_bytes;
  int v_pad;                // V rounded up to the vocab tile
  float* logits;            // optional [M][V]
  float* conf;              // [M]
  int32_t* token;           // [M]
  int m_pad;
  int emit;                 // nonzero: the screen writes the raw product to zpart [M][v_pad] and stops
  int prepacked;            // nonzero: hhi (and hlo) already hold rows 0..M-1 (no k_pack); rows
                            // M..m_pad-1 hold finite values that only reach their own logits
  // Fused unmasking in a pre-generated order (k_decide): with cand_pos != NULL,
  // row m = (b, c) is unmasked at position cand_pos[b*cand_stride + c]:
  // seq_tokens[b][pos] = its token (when seq_tokens != NULL).
  const int32_t* cand_pos;
  int64_t cand_stride;
  int32_t* seq_tokens;
  int* err;
  // Decision certificate: wmax = max_v ||W_v||_2 (rounded up, built at init);
  // trace (optional) [M][8] = {z_best, i_best, z_runner_up, i_runner_up, D, eps_s,
  // eps_e, flags} per row (int fields as bit patterns); stats (optional) counts
  // rows that re-scored beyond the candidates, rows that re-scored whole tiles
  // and rows whose two best exact logits lie within 2 eps_e.
  const float* wmax;
  float* trace;
  unsigned* stats;
  int n_split;              // set by the launcher: hidden splits summed before the epilogue
};
hipError_t launch_vocab(const Geometry& g, const VocabArgs& a, hipStream_t s);
// max_v ||W_v||_2 of the vocabulary head, rounded up, into *out (which must hold 0)
hipError_t launch_row_norm_max(const Geometry& g, const void* w, float* out, hipStream_t s);
// The tiled copy of a bf16 W described at VocabArgs::wt (built at init).
hipError_t launch_tile_w(const Geometry& g, const void* w, uint16_t* wt, hipStream_t s);
inline size_t tiled_w_elems(int V, int hidden) { return ((size_t)(V + 511) / 512) * 512 * (size_t)hidden; }
// Vocabularies from which the tiled copy is kept: where the wide screen runs
// with a single row tile (W, not h, is the stream that bounds it).
constexpr int kTiledWMinVocab = 32768;

// Upper layers: y = h_prev W^T for every query row (h_prev fp32, split into
// bf16 hi + lo; W bf16 [N][hidden] with N = (H + 2 H_kv) d, rows q | k | v),
// then RoPE at the row's position and scatter: q of every row to qbuf
// [B][H][qbuf_rows][d]; k and v of the D rows into the layer's cache at slot
// slot0 + r (keys [B][H_kv][slots][d], values transposed in 64-slot tiles);
// k and v of the C|R rows (index j = r - n_d) to tk [B][H_kv][t_pad][d] and
// tvt [B][H_kv][d][t_pad].
struct ProjArgs {
  const void* w;
  const float* h;
  int64_t h_stride;
  int n_d, n_c, n_q;        // n_q = n_d + n_c + R rows per sequence
  const int32_t* d_pos;
  int64_t d_stride;
  const int32_t* c_pos;
  int64_t c_stride;
  uint16_t* hhi;            // [m_pad][hidden]
  uint16_t* hlo;
  float* z;                 // [m_pad][n_pad]
  int n_pad;                // N rounded up to the vocab tile
  const float* rope_cos;
  const float* rope_sin;
  void* qbuf;
  int qbuf_rows;
  void* kc;
  void* vc;
  int slot0;
  void* tk;
  void* tvt;
  int t_pad;
  int* err;
};
hipError_t launch_project(const Geometry& g, const ProjArgs& a, hipStream_t s);
hipError_t launch_rope_scatter(const Geometry& g, const ProjArgs& a, int M, hipStream_t s);

struct SelectArgs {
  const int32_t* cand_pos;
  int64_t cand_stride;
  const float* conf;
  const int32_t* token;
  int n_cand, n_select, by_conf;
  int32_t* out_tok;
  int32_t* out_pos;
  int32_t* rem_pos;
  int32_t* seq_tokens;
  int* err;
};
hipError_t launch_select(const Geometry& g, const SelectArgs& a, hipStream_t s);

hipError_t launch_fill_i32(int32_t* p, int32_t v, int n, hipStream_t s);

// Training-form (block-mask) attention, bf16 in, fp32 out, head_dim 128.
constexpr int kBlockAttnMaxTiles = 256;   // rows per sequence <= 256 * 64
struct BlockAttnArgs {
  const void* q;            // bf16 [B][n][H][128]
  const void* k;            // bf16 [B][n][H_kv][128]
  const void* v;            // bf16 [B][n][H_kv][128]
  const int32_t* blk;       // [B][n] block id of every row
  const int32_t* n_clean;   // [B] number of clean blocks M
  float* out;               // [B][n][H][128]
  int32_t* ranges;          // workspace [B][ceil(n/64)][2]
  int B, n, H, Hkv;
  int nbk, real_blocks;     // set by the launcher
};
hipError_t launch_block_attention(BlockAttnArgs a, hipStream_t s);

// The library-owned range array of the allocation-free block attention:
// kStaticRangeInts int32 per GPU; *ptr = its device address on the current device.
constexpr int kStaticRangeInts = 16384;
hipError_t block_attention_static_scratch(int32_t** ptr, size_t* n_ints);

}  // namespace mdm
