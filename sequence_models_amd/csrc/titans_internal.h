// Internal interface between the C-ABI layer and the HIP kernels of libtitans_mem.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "titans_mem.h"

namespace titans {

// Everything a scan or retrieve launch needs, already validated on the host.
struct ScanArgs {
    int64_t B, T, H;
    int C;
    int io;                    // titans_dtype
    int L;
    int n[TITANS_MAX_LAYERS + 1];
    int64_t P;
    int64_t off[TITANS_MAX_LAYERS + 2];  // float offset of W_l inside one memory, l = 1..L
    int64_t qs[3], ys[3], gs[3], ss[2], s0s[2];
    const void* q;
    const void* k;
    const void* v;
    const float* alpha;
    const float* eta;
    const float* beta;
    const float* theta0;
    const float* s0;
    void* y;
    float* surprise;           // NULL, or [B, T, H] per-token gradient norms (gate strides)
    float* thetaT;
    float* sT;
    void* ws;
    int debug;                 // test hooks (0 in normal use), see abi.hip
    int sides;                 // pair path: workgroups per memory (4, else 2), set by the dispatcher
    int bias;                  // titans_bias of the writes
    float bias_param;          // Huber delta or l_p exponent
};

// The reverse pass: the forward problem plus output cotangents and the input cotangents
// it writes (q/k/v cotangents in q's layout and dtype, gate cotangents in the gates'
// layout, state cotangents with the theta_T / s_T strides).
struct BwdArgs {
    ScanArgs a;
    const void* dy;         // y's layout (a.ys)
    const float* dthetaT;   // NULL: zero
    const float* dsT;       // NULL: zero
    void* dq;
    void* dk;
    void* dv;
    float* dalpha;
    float* deta;
    float* dbeta;
    float* dtheta0;
    float* ds0;
};

// Reverse-mode derivatives of the scan, one workgroup per (b, h): a forward sweep stores
// every chunk's start state in the workspace, then a reverse chunk loop recomputes each
// chunk and runs its adjoint (products on fp32 FMAs).
size_t scan_backward_workspace_bytes(const ScanArgs& a);
hipError_t launch_scan_backward(const BwdArgs& b, hipStream_t stream);

// Generic chunked scan: any supported shape, one workgroup per (b, h), per-chunk
// intermediates in the workspace.  Its matrix products run on bf16 MFMA (fp32
// accumulation) for bf16 I/O and on fp32 FMAs for fp32 I/O; state is fp32 either way.
size_t scan_generic_workspace_bytes(const ScanArgs& a);
hipError_t launch_scan_generic(const ScanArgs& a, hipStream_t stream);

// Linear memory (L = 1) with the squared-error bias: the chunk carries are affine maps of
// [W | S], composed per group of chunks in parallel, chained over the groups, then every
// group's chunks run from its start state in parallel (three launches).
bool scan_linear_supported(const ScanArgs& a);
size_t scan_linear_workspace_bytes(const ScanArgs& a);
hipError_t launch_scan_linear(const ScanArgs& a, hipStream_t stream);

// The generic scan as a chain of GPU-wide launches (4L - 2 per chunk), each spreading
// one step's matrix products over 64 x 64 tiles of every memory; for wide memories.
size_t scan_phased_workspace_bytes(const ScanArgs& a);
hipError_t launch_scan_phased(const ScanArgs& a, hipStream_t stream);

// Fused MFMA scan for the 64 -> 256 -> 64 memory, C = 64, bf16 I/O: one workgroup per
// (b, h), state resident in registers, no workspace.
bool scan_mfma_supported(const ScanArgs& a);
hipError_t launch_scan_mfma(const ScanArgs& a, hipStream_t stream);

// Fused MFMA scan split over pairs (a.sides = 2) or quads (a.sides = 4) of workgroups
// (same shape as above): each (b, h) memory is served by that many workgroups on one XCD
// that exchange partial sums through the workspace; cooperative launch of
// scan_pair_workgroups(a) workgroups.  The per-token surprise needs pairs.
bool scan_pair_supported(const ScanArgs& a);
size_t scan_pair_workspace_bytes(const ScanArgs& a);
int64_t scan_pair_workgroups(const ScanArgs& a);
// Extra workspace of a pair-path call that also writes the per-token surprise norms.
size_t scan_pair_surprise_bytes(const ScanArgs& a);
hipError_t launch_scan_pair(const ScanArgs& a, hipStream_t stream);
// The pair path without a caller workspace: a static device array of
// scan_pair_scratch_capacity() bytes per GPU (scan_pair_scratch: its address on the current
// device, looked up once per device).  A call needs scan_pair_scratch_exchange_bytes for the
// exchange areas plus scan_pair_scratch_chunk_bytes per gradient chunk of C tokens it
// covers (the coefficient records).
size_t scan_pair_scratch_capacity();
hipError_t scan_pair_scratch(void** ptr);
size_t scan_pair_scratch_exchange_bytes(const ScanArgs& a);
size_t scan_pair_scratch_chunk_bytes(const ScanArgs& a);

// Generic retrieve: any supported shape, products as in the generic scan.
hipError_t launch_retrieve_generic(const ScanArgs& a, hipStream_t stream);

// MFMA retrieve for any memory with widths multiples of 16 (<= 512) and bf16 q / y:
// activations in LDS, weights streamed in windows.
bool retrieve_wide_supported(const ScanArgs& a);
hipError_t launch_retrieve_wide(const ScanArgs& a, hipStream_t stream);

// MFMA retrieve for the 64 -> 256 -> 64 memory with bf16 q / y; cus = compute units of
// the device (sets the tokens per workgroup).
bool retrieve_mfma_supported(const ScanArgs& a);
int retrieve_mfma_tiles(const ScanArgs& a, int64_t cus);
hipError_t launch_retrieve_mfma(const ScanArgs& a, int64_t cus, hipStream_t stream);

// MAG block (memory as gate): the front-end projection and gates, the gated
// sliding-window attention and the output projection around one memory scan.  Shapes
// are validated by the ABI layer; the pointers after b_gate/w_out are workspace pieces
// placed by mag_place.
struct MagArgs {
    int64_t B, T, H;
    int d;                 // head width (the memory's input and output width)
    int window;            // attention window, the token itself included
    float eta_scale;
    const __bf16* x;       // [B, T, D], D = H d
    const __bf16* w_in;    // [3D + 3H, D]
    const float* b_gate;   // [3H]
    const __bf16* w_out;   // [D, D]
    __bf16* out;           // [B, T, D]
    int64_t ldp;           // row pitch of proj (3D + 3H rounded up to a multiple of 4)
    float* proj;           // [B T, ldp] fp32
    __bf16 *q, *k, *v, *ymem, *o;  // [B, T, H, d]
    float *alpha, *eta, *beta;     // [B, T, H]
};
bool mag_head_dim_supported(int d);
size_t mag_workspace_bytes(const MagArgs& g);
void mag_place(MagArgs& g, void* ws);
hipError_t launch_mag_front(const MagArgs& g, hipStream_t stream);
hipError_t launch_mag_attention(const MagArgs& g, hipStream_t stream);
hipError_t launch_mag_out(const MagArgs& g, hipStream_t stream);
// MAC block attention for the segment of tokens row0 .. row0 + len - 1: every query sees
// the segment's memory reads h (a [B, T, H, d] buffer, rows of the segment) as a prefix of
// keys and values and its own segment's keys causally; writes g.o for those rows.
hipError_t launch_mac_attention(const MagArgs& g, const __bf16* h, int64_t row0, int64_t len,
                                hipStream_t stream);

}  // namespace titans
