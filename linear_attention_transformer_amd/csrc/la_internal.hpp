// la_internal.hpp -- calls shared by the library's own translation units and
// not exported: la_forward / la_backward with the outputs written in a given
// layout, so that the layer (la_layer.hip) can have the attention write its
// output rows straight into the layout its projections take.
#pragma once

#include <cstddef>
#include <cstdint>

namespace la_internal {

// element (b, h, n, d) of an output at b * sb + h * sh + n * sn + d
struct OutStrides {
    int64_t sb, sh, sn;
};

// la_forward (no den, optional saved state) with O in layout `o`
__attribute__((visibility("hidden"))) int forward_to(const void *Q, const void *K,
                                                     const void *V, void *O, int64_t B,
                                                     int64_t H, int64_t N, int64_t D, int causal,
                                                     int dtype, void *state_out, void *ws,
                                                     size_t ws_bytes, void *stream,
                                                     OutStrides o);

// la_backward with dQ, dK, dV in layout `o` (their elements may interleave)
__attribute__((visibility("hidden"))) int backward_to(const void *Q, const void *K,
                                                      const void *V, const void *dO, void *dQ,
                                                      void *dK, void *dV, int64_t B, int64_t H,
                                                      int64_t N, int64_t D, int causal,
                                                      int dtype, const void *state_in, void *ws,
                                                      size_t ws_bytes, void *stream,
                                                      OutStrides o);

}  // namespace la_internal
