// The state walk and the Gram pass in one launch.
//
// The first nwalk workgroups walk (walk_block), the rest form the causal Gram
// tiles (gram_block, without dt prep, which is launched before: the walk needs
// dt and the cumulative sums, the Gram tiles are read only by later calls).
// The walk runs one eight-wave workgroup per CU, bound by load latency and LDS
// more than by issue, so the Gram workgroups dispatched after it share its CUs
// and use the issue slots it leaves.  Both halves use 512-thread workgroups (two
// heads per walk workgroup, 256-token chunks); other shapes launch the two
// kernels one after the other.
#pragma once

#include <type_traits>

#include "gram.h"
#include "state_walk.h"

namespace ssd {

template <typename T, int P, int N, int Q, bool BWD, bool SEQ, bool TRANS>
__global__ void __launch_bounds__(512, 4) k_walk_gram(Dims d, SegTab tab, WalkArgs<T> wa,
                                                     int64_t nwalk, int S, const T* __restrict__ bc,
                                                     int64_t bstr, T* __restrict__ gram) {
    constexpr int LW = walk_lds<T, P, N, 2>(), LG = gram_lds<T, N, Q>();
    __shared__ __attribute__((aligned(16))) T lds[LW > LG ? LW : LG];
    if ((int64_t)blockIdx.x < nwalk)
        walk_block<T, P, N, BWD, SEQ, 2>(d, tab, wa, lds, blockIdx.x, nwalk);
    else
        gram_block<T, N, Q, TRANS>(d, S, bc, bstr, gram, lds, blockIdx.x - nwalk, gridDim.x - nwalk,
                                   false, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                   nullptr);
}

// True where the combined launch applies (both halves 512 threads).
template <typename T>
inline bool walk_gram_fits(const Dims& d) {
    return walk_heads<T>(d) == 2 && d.Q == 256;
}

// The walk of `wa` and the Gram tiles of (bc, bstr) into `gram`, in one launch.
template <typename T, int P, int N, bool BWD, bool TRANS>
inline hipError_t launch_walk_gram(const Dims& d, const SegTab& t, const WalkArgs<T>& wa,
                                   const T* bc, int64_t bstr, T* gram, hipStream_t s) {
    if constexpr (!std::is_same<T, bf16>::value) {
        return hipErrorInvalidValue;  // float32 walks one head per workgroup
    } else {
        if (!walk_gram_fits<T>(d)) return hipErrorInvalidValue;
        const int64_t nwalk = (int64_t)(d.H / 2) * wa.sp.n * d.batch;
        const int S = gram_split(d);
        const int64_t ngram = (int64_t)d.nchunk * d.G * d.batch * S;
        const dim3 grid((unsigned)(nwalk + ngram)), block(512);
        if (wa.seq)
            return launch(k_walk_gram<T, P, N, 256, BWD, true, TRANS>, grid, block, s, d, t, wa,
                          nwalk, S, bc, bstr, gram);
        return launch(k_walk_gram<T, P, N, 256, BWD, false, TRANS>, grid, block, s, d, t, wa,
                      nwalk, S, bc, bstr, gram);
    }
}

}  // namespace ssd
