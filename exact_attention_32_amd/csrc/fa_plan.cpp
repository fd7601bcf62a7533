// fa_plan.cpp -- host-side launch planning shared by the C ABI (workspace
// sizes) and the decode launcher: how the key axis of a decode call is cut
// into chunks.  Plain host code (no device code, no HIP runtime calls).
#include <algorithm>

#include "fa_internal.h"

namespace fa {

int decode_num_splits(int B, int H, int Nq, int Nk, int requested) {
    const long smax = (Nk + kDecodeMinChunk - 1) / kDecodeMinChunk;
    if (requested > 0) return (int)std::min<long>(requested, smax);
    // About the target number of single-wave workgroups in all, chunks of at
    // least kDecodeMinChunk keys.
    const long target = Nq > kDecodeValuQueries ? kDecodeTargetWavesMfma : kDecodeTargetWaves;
    const long bh = (long)B * H;
    long s = (target + bh - 1) / bh;
    if (s > smax) s = smax;
    if (s < 1) s = 1;
    return (int)s;
}

int decode_chunk(int Nk, int S, int granule) {
    const int c = (Nk + S - 1) / S;
    return (c + granule - 1) / granule * granule;
}

}  // namespace fa
