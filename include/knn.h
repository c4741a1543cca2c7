/*
 * knn.h -- C ABI of the k-nearest-neighbour sparse atom-pair encoder in
 * libtriattn.so (MI355X, gfx950).
 *
 * What is computed (Design-CP summary, implementation details, memory
 * optimisation: in low-memory mode the atom-pair tensor P is built only at the
 * sparse indices of each atom's k nearest neighbours, never for all L x L atom
 * pairs).  The page does not print the features; this library computes:
 *   N(l)  = the k atoms m != l of smallest squared distance to atom l, in
 *           ascending order, equal distances to the lower index.  The squared
 *           distance is float32 ((dx*dx + dy*dy) + dz*dz), d = x_l - x_m, every
 *           operation rounded to nearest even, none fused;
 *   p_lm  = W_l s_l + W_m s_m + W_d phi(x_l - x_m),
 *           phi(d) = (d_x, d_y, d_z, 1 / (1 + |d|^2)) with |d|^2 the selection
 *           value -- the projected single features of both atoms, their
 *           relative position and an inverse-square distance, the feature set
 *           of AlphaFold 3's atom-pair embedding (Abramson et al. 2024,
 *           Algorithm 5).  Accumulated in float32, stored bfloat16 (nearest even).
 *
 * Conventions (as in include/triattn.h): DEVICE pointers, 16-byte aligned,
 * dense row-major; weights in torch.nn.Linear layout W[out][in]; the caller
 * owns every buffer; the library never allocates, frees or synchronises; every
 * argument is validated on the host before anything is enqueued (return codes
 * of include/triattn.h; on error nothing is launched and no output touched).
 * Coordinates must be finite: with a non-finite one the selection is
 * unspecified (a slot no atom fills holds index -1).
 */
#ifndef KNN_H
#define KNN_H

#include <stddef.h>
#include <stdint.h>

#include "triattn.h"

#ifdef __cplusplus
extern "C" {
#endif

#define KNN_SINGLE_CHANNELS 128 /* c_s */
#define KNN_PAIR_CHANNELS 16    /* c_p */
#define KNN_MAX_K 64
#define KNN_MAX_ATOMS (1 << 24)

/* Workspace bytes knn_pair_encode needs for L atoms (host only).
 * Errors: TA_ERR_NULL_PTR (bytes NULL), TA_ERR_BAD_SHAPE (L < 0 or L > KNN_MAX_ATOMS). */
int knn_workspace_bytes(int64_t L, size_t* bytes);

/* Neighbour lists and pair features of L atoms.
 *   x     fp32 [L][3]        coordinates
 *   s     bf16 [L][128]      single features
 *   w_l   bf16 [16][128]     projection of the query atom's features
 *   w_m   bf16 [16][128]     projection of the neighbour's features
 *   w_d   fp32 [16][4]       projection of phi
 *   nbr   int32 [L][k]       out: N(l), ascending distance
 *   pair  bf16 [L][k][16]    out: pair[l][n] = p_{l, nbr[l][n]}
 *   ws    at least knn_workspace_bytes(L) bytes (contents on entry ignored)
 * Requires 1 <= k <= KNN_MAX_K and, for L >= 1, k <= L - 1; L = 0 enqueues
 * nothing.  Errors: TA_ERR_BAD_SHAPE (L or k out of range), TA_ERR_NULL_PTR,
 * TA_ERR_MISALIGNED, TA_ERR_WORKSPACE_TOO_SMALL, TA_ERR_ALIAS (nbr, pair and ws
 * overlap one another or an input), TA_ERR_HIP (launch rejected). */
int knn_pair_encode(const float* x, const void* s, int64_t L, int k, const void* w_l, const void* w_m,
                    const float* w_d, int32_t* nbr, void* pair, void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KNN_H */
