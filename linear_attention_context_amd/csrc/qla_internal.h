// qla_internal.h -- declarations shared by the host entry points and the
// kernel launchers of libqla.so (not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>

#include "qla.h"

namespace qla {

struct LaunchArgs {
    const float* H;
    const float* M;
    const float* S0;  // may be null: zero initial state
    float* out;
    int layout;
    int direction;
    long long chains;  // batch * heads
    int heads;
    int n_seg;
    int K;
    int V;
    void* stream;
    int cus;  // compute units of the device (a K <= 128 workgroup occupies one CU)
};

// Head-group table copied by value into the grouped kernel's arguments.
// variant = 2 * layout + direction.
struct GroupTable {
    int n;
    int begin[QLA_MAX_GROUPS];
    int count[QLA_MAX_GROUPS];
    int variant[QLA_MAX_GROUPS];
};

// Segment offsets of a variable-length call, copied by value into the
// kernel's arguments: sequence b has offs[b+1] - offs[b] segments.
struct SeqTable {
    int n;
    int offs[QLA_MAX_SEQS + 1];
};

int tiles_for(int V);
// Largest workgroup any kernel of the library launches (threads).
int max_threads_per_group();
hipError_t launch_correct_h0(const LaunchArgs& a);
hipError_t launch_correct_h0_grouped(const LaunchArgs& a, const GroupTable& table);
hipError_t launch_correct_h0_varlen(const LaunchArgs& a, const SeqTable& seqs);
// Whether a plain call of this shape runs two tiles per workgroup on a
// device with `cus` compute units.
bool plain_call_pairs_tiles(int K, long long chains, int V, int n_seg, int cus);

}  // namespace qla
