// Internal declarations shared by the host and device translation units of libtq.
#ifndef TQ_INTERNAL_H_
#define TQ_INTERNAL_H_

#include <stddef.h>
#include <stdint.h>

#include "tq.h"

namespace tq {

// Records a message for tq_last_error() and returns `status`.
int fail(int status, const char* fmt, ...);
int ok();

// Float offsets into a codebook table (all bit widths of one kind).
constexpr int centroid_offset(int bits) { return (1 << bits) - 2; }
constexpr int boundary_offset(int bits) { return 510 + (1 << bits) - bits - 1; }
// Quantiser lookup grids: per bit width a header {S, O, n_bins, entry offset}
// at kLutHeaderOffset + 4 (bits - 1); entries {base (u32), boundary (f32)}.
constexpr int kLutHeaderOffset = 1024;
// Pair tables of widths 1..4 (float2 entries; width b starts at entry
// pair_offset_host(b) = 0, 4, 20, 84), then the lookup grids' entries.
constexpr int kPairOffset = 1056;
constexpr int pair_offset_host(int b) { return b == 1 ? 0 : b == 2 ? 4 : b == 3 ? 20 : 84; }
constexpr int kLutEntriesOffset = kPairOffset + 2 * 340;
constexpr int kLutMaxBins = 1400;
// PolarQuant tables: the angle shift t (radius b - t bits, angle b + t bits at
// page width b) as a float in the table's last entry (0 for an even split).
constexpr int kPolarShiftSlot = TQ_CODEBOOK_TABLE_FLOATS - 1;
constexpr int kLutByteBins = 256;   // grids this small are indexed by a saturating byte conversion

// Decode split-K geometry.
constexpr int kDecodeWaves = 4;             // waves per split workgroup
constexpr int kTargetSplitGroups = 1024;    // workgroups the split grid aims for
constexpr int kLongRangePages = 64;         // common ranges longer than this are cut further
constexpr int kMaxPagesPerSplit = 256;      // a range's descriptors fit the workgroup's LDS copy
constexpr int kQPrepFloats = 3 * 128;       // rotated q, plain q, S q (all pre-scaled)
constexpr int kPartialFloats = 4 + 128;     // m, l, (pad), acc[128]
constexpr int kMaxPartials = 7168;          // partials per (session, query head), all classes (1024 + 4096 + 2048)

// Split-K geometry: the common class (1-4 bit codebook pages without QJL)
// covers the page table in ranges of pages_per_split pages; the other class
// (fp16, QJL, mixed widths: heavier per page, two waves per SIMD) in ranges
// half as long, and the wide class (5-8 bits) in ranges a quarter as long (one
// page per wave: its pages are few, and latency-bound).
struct SplitPlan {
  int n_splits;
  int pages_per_split;
  int n_splits_general;         // the other class (fp16, QJL, mixed widths)
  int pages_per_split_general;
  int n_splits_wide;            // the wide class (5-8 bits)
  int pages_per_split_wide;
  bool cut;                     // common ranges cut for a long context
  int min_pages_per_split_wide; // the shortest wide ranges a launch may choose
  int max_splits_wide;          // and their count (the workspace's wide partials)
};
// Time of a wide page in common pages, for balancing a merged launch's ranges.
constexpr float kWidePageCost = 1.5f;
SplitPlan split_plan(int n_sessions, int n_kv_heads, int max_pages);
size_t decode_workspace_bytes(int n_sessions, int n_q_heads, const SplitPlan& sp);

// Each HIP translation unit's device check word (checked builds): OR-ed into
// *out, zeroed when reset.
int check_word_encode(uint32_t* out, bool reset);
int check_word_pages(uint32_t* out, bool reset);
int check_word_decode(uint32_t* out, bool reset);
int check_word_dequant(uint32_t* out, bool reset);

// Validation shared by the device entry points (host only, before any HIP call).
int check_layer(const tq_layer* layer);
int check_cache(const tq_cache* cache);

}  // namespace tq

#endif  // TQ_INTERNAL_H_
