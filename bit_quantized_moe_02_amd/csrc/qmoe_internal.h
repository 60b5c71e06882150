// Internal declarations shared by the host and device translation units of
// libqmoe.  Not part of the public ABI (include/qmoe.h).
#pragma once

#include <stdint.h>

#include <string>

namespace qmoe {

// Records the message moe_last_error() returns on this thread and passes
// `code` through, so call sites can write `return fail(MOE_ERR_..., "...")`.
int fail(int code, const std::string& msg);
void clear_error();

// Tile geometry (see include/qmoe.h): 16 rows x 256 columns per tile.
constexpr int kTileRows = 16;
constexpr int kTileCols = 256;

inline int64_t pad256(int64_t k) { return (k + 255) / 256 * 256; }

// Bytes of one tile of each format; 0 for an unknown format.
int tile_bytes(int fmt);

}  // namespace qmoe

struct moe_weights;

namespace qmoe {

// Shape, format and pointer checks of a weight set (those of the decode and
// prefill calls); MOE_OK or the failing code with its message recorded.
int validate_weights(const moe_weights* w, const char* fn);

// Measurement hook (moe_profile_next_launch): pending (kernel id, start
// event, stop event) entries of this thread; each is consumed by the next
// launch of its kernel.
struct ProfileHook {
  static constexpr int kMax = 8;
  int n = 0;
  int kernel_id[kMax];
  void* start[kMax];
  void* stop[kMax];
};
ProfileHook& profile_hook();

}  // namespace qmoe
