// bi_plan.h -- the recipe table and the launch plan (host only).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "bi.h"

namespace bi {

enum Path { kPathDecode = 1, kPathPersistent = 2, kPathDecodeWg = 3, kPathDecodeDma = 4, kPathDecodeXcd = 5 };

// Every workspace starts with a region of kDecodeCounterBytes that holds the
// arrival counters of the one-launch decode (one 32-bit counter per
// output-tile group, each on its own 128-byte line).  It must be zero when a
// workspace is first used; no call writes anything else there, and every call
// leaves the counters at zero.  Tile partials and MoE intermediates follow it.
constexpr int kDecodeMaxCounters = 128;
constexpr size_t kDecodeCounterBytes = 16384;

// Most tile partials the one-launch decode kernel keeps in LDS (64 KiB).
constexpr int kDecodeWgMaxTiles = 64;

// Persistent-kernel tiling: a workgroup computes a BM x BN output tile with
// WM x WN waves.  Tiling never changes the numerics.
struct Tiling {
    int bm, bn, wm, wn;
};

// A measured entry of the key table (written by the offline sweeper,
// deterministic_persistent_gemm_amd/sweep.py, into bi_table.inc).  block_k
// is part of the recipe; every other field only picks kernel shapes.
struct KeyEntry {
    int32_t dtype;
    int64_t N, K;
    int32_t block_k;        // recipe: width of one k tile partial
    int32_t m_decode_max;   // largest M on a decode kernel
    int32_t decode_path;    // BI_PATH_DECODE, _DECODE_WG or _DECODE_DMA (0: automatic)
    // persistent tile codes (0: automatic): tile_a for M <= m_a, tile_b for
    // m_a < M <= m_b, tile_c above
    int64_t m_a;
    int32_t tile_a;
    int64_t m_b;
    int32_t tile_b, tile_c;
    int32_t m_xcd_max;      // largest M on the XCD hand-over decode (0: never); below
                            // m_decode_max it takes precedence over decode_path
};

// The table entry of a key, or nullptr.
const KeyEntry* table_lookup(int32_t dtype, int64_t N, int64_t K);

// Number of entries in the compiled table and the i-th one (for checks).
int table_size();
const KeyEntry* table_entry(int i);

struct Plan {
    bi_recipe_t recipe;
    int path;
    int kbpt;        // k blocks (of 32) per tile partial = block_k / 32
    int tiles_k;     // tile partials per output element = K / block_k
    int mtiles;      // 16-row tiles of M (decode path)
    int ntiles;      // 16-column tiles of N (decode path)
    Tiling tiling;   // persistent path
    int tile_code;   // persistent tile shape, 0 = automatic (table entry or heuristic)
    int m_per_wave;  // decode paths: 16-row M tiles one wave carries (1, 2, 4), 0 = automatic
    int ksplit;      // persistent tile codes 28, 29: workgroups per output tile (0: unsplit)
    size_t ws_bytes; // workspace the plan needs (decode or k-split tile partials)
};

// The recipe of a key -- a pure function of (dtype, N, K).
bi_status_t recipe_for(int32_t dtype, int64_t N, int64_t K, bi_recipe_t* out);

// Checks a recipe is one the kernels can carry out for this (N, K).
bi_status_t recipe_valid(const bi_recipe_t& r, int64_t N, int64_t K);

// Internal request bit of make_plan: serve the ring-fed fp32 tiles unsplit
// (tile codes 28, 29 run as 23, 24 and need no workspace); same bits, for a
// caller whose workspace is capped.
constexpr int32_t kPathNoSplit = 1 << 16;

// Picks the kernel path and its shape for M rows.  path_req: BI_PATH_*.
bi_status_t make_plan(const bi_recipe_t& r, int32_t path_req, int64_t M, int64_t N, int64_t K,
                      Plan* plan);

// Persistent tile shapes selectable through the experiment entry point.
bool tile_code_valid(int dtype, int code);

// Whether the direct-to-LDS decode kernel serves this plan (bi_linear.hip).
bool decode_dma_ok(const Plan& p, int64_t K);

// M tiles one decode wave carries (bi_linear.hip): the two-launch decode
// shares W fragments over 2 or 4 M tiles at large M; the XCD hand-over keeps
// one M tile per wave while the counters allow it, since its last wave folds
// the M tiles of its group one after the other.
int decode_m_per_wave(const Plan& p);
int xcd_m_per_wave(const Plan& p);

// Whether the one-launch decode serves this plan: several k tiles, N/16 a
// multiple of 8 (so every wave of an output tile runs on one XCD), and no
// more output-tile groups than there are counters.
bool decode_xcd_ok(const Plan& p);

// The k split of the ring-fed fp32 tiles (tile codes 28, 29; bi_linear.hip):
// workgroups per output tile (0: no split serves this plan), the k tiles
// worked on at once, the tile rows, the tile count and the workspace.
struct RingSplit {
    int ksplit, par, bm, tiles;
    size_t ws_bytes;
};
RingSplit ring_split_plan(const Plan& p, int64_t M, int64_t N, int64_t K, int code);

// Number of compute units of the current device (cached per device).
int device_cu_count();

}  // namespace bi
