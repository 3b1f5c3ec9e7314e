// Sizes of the records of the full-sort solver ("Fast LapSum: Exact
// Differentiable Top-k at Million Scale", section 2.2) that the host lays out
// in the workspace.  The solver itself lives in segment_dev.hpp and
// bucket_dev.hpp: full rows run through the bucketed kernels of band.hip, and
// a row whose bracket missed is solved exactly by one workgroup
// (fallback_row) at the end of its band kernel: when every bracket held it
// costs nothing; on a miss it is slower but exact and deterministic.
#include "segment_dev.hpp"

namespace lapsum {

size_t tile_agg_bytes() { return sizeof(TileAgg); }
size_t pre_bytes() { return sizeof(Pre); }
size_t suf_bytes() { return sizeof(Suf); }

}  // namespace lapsum
