// Internal launcher interface between the C ABI (abi.cpp) and the kernels.
// Arguments are validated by the caller; these only enqueue work on `stream`.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

// Instantiates FN<T, D, M> for the built (D, M) set {32, 64} x {32, 64}.
#define LA_DISPATCH_DM(FN, T, ...)                \
  switch (D * 100 + M) {                          \
    case 3232: return FN<T, 32, 32>(__VA_ARGS__); \
    case 3264: return FN<T, 32, 64>(__VA_ARGS__); \
    case 6432: return FN<T, 64, 32>(__VA_ARGS__); \
    case 6464: return FN<T, 64, 64>(__VA_ARGS__); \
    default: return hipErrorInvalidValue;         \
  }

namespace la {

// Tokens per sequence block of the causal / non-causal kernels.
int causal_block_tokens(int BH, int N);
size_t causal_ws_bytes(int BH, int N, int D, int M, int bf16);
size_t noncausal_ws_bytes(int BH, int N, int D, int M, int bf16);

hipError_t launch_causal(const void* q, const void* k, const void* v, void* o, int BH, int N, int D, int M,
                         int bf16, const float* S0, const float* z0, float* S_out, float* z_out, void* ws,
                         hipStream_t stream);
// Single-pass bf16 causal path (one launch).
size_t causal_fused_ws_bytes(int BH, int N, int D, int M);
hipError_t launch_causal_fused(const void* q, const void* k, const void* v, void* o, int BH, int N, int D, int M,
                               const float* S0, const float* z0, float* S_out, float* z_out, void* ws,
                               hipStream_t stream);
// Single-pass float32 causal kernel (causal_fused32.hip).
size_t causal_fused32_ws_bytes(int BH, int N, int D, int M);
hipError_t launch_causal_fused32(const void* q, const void* k, const void* v, void* o, int BH, int N, int D, int M,
                                 const float* S0, const float* z0, float* S_out, float* z_out, void* ws,
                                 hipStream_t stream);
hipError_t launch_noncausal(const void* q, const void* k, const void* v, void* o, int BH, int N, int D, int M,
                            int bf16, void* ws, hipStream_t stream);
// bf16 non-causal path (state, reduce and apply kernels).
size_t noncausal_bf16_ws_bytes(int BH, int N, int D, int M);
hipError_t launch_noncausal_bf16(const void* q, const void* k, const void* v, void* o, int BH, int N, int D, int M,
                                 void* ws, hipStream_t stream);
// Softmax attention decode step over a key/value cache (the comparison baseline):
// appends k, v at row L of Kc [BH][Lmax][D], Vc [BH][Lmax][M] and attends over rows 0..L.
hipError_t launch_softmax_decode(const void* q, const void* k, const void* v, void* o, void* Kc, void* Vc, int BH,
                                 int L, int Lmax, int D, int M, int bf16, hipStream_t stream);
// Per-block state increments for bf16 inputs on bf16 MFMA (phi(K) as head and tail):
// agg [BH][nblk][D][M], aggz [BH][nblk][D], blocks of tblk tokens.
hipError_t launch_block_state_bf16(const void* k, const void* v, int BH, int N, int D, int M, int tblk, int nblk,
                                   float* agg, float* aggz, hipStream_t stream);
// Exclusive per-block prefix states (S, z) from a zero initial state (backward pass).
hipError_t launch_block_prefix(const void* k, const void* v, int BH, int N, int D, int M, int bf16, int tblk,
                               int nblk, float* agg, float* aggz, hipStream_t stream);
// Backward of causal linear attention.
size_t causal_bwd_ws_bytes(int BH, int N, int D, int M);
hipError_t launch_causal_bwd(const void* q, const void* k, const void* v, const void* dO, void* dq, void* dk,
                             void* dv, int BH, int N, int D, int M, int bf16, void* ws, hipStream_t stream);
// bf16 backward kernels, given the block prefix states (preS, preZ) and room
// for 1/den and b per token and the per-block suffix states.
hipError_t launch_causal_bwd_bf16(const void* q, const void* k, const void* v, const void* dO, void* dq, void* dk,
                                  void* dv, int BH, int N, int D, int M, int tblk, int nblk, float* preS, float* preZ,
                                  float* inv, float* b, float* suf, hipStream_t stream);
// In-place exclusive suffix sums of per-block records of SZ floats (fixed order).
hipError_t launch_suffix_scan(float* suf, int BH, int nblk, int SZ, hipStream_t stream);
// Block scan of state records [BHs][nblk][DM] / [BHs][nblk][D]: exclusive prefix in
// place when exclusive != 0, starting from (S_init, z_init) (NULL: zero); the
// totals go to (S_tot, z_tot) when non-NULL.
hipError_t launch_state_scan(float* agg, float* aggz, int BHs, int nblk, int DM, int D, const float* S_init,
                             const float* z_init, float* S_tot, float* z_tot, int exclusive, hipStream_t stream);
// (S_out, z_out) <- (S_init, z_init), or zeros when S_init is NULL.
hipError_t launch_state_copy(const float* S_init, const float* z_init, float* S_out, float* z_out, long long nS,
                             long long nz, hipStream_t stream);
// Linear attention with another feature map (map 1..3 = DPFP-nu, 4 = degree-2
// polynomial), causal or not; feature dimension and workspace.
int featmap_dim(int map, int D);
size_t featmap_ws_bytes(int map, int BH, int N, int D, int M);
hipError_t launch_featmap(int map, const void* q, const void* k, const void* v, void* o, int BH, int N, int D,
                          int M, int bf16, int causal, const float* S0, const float* z0, float* S_out, float* z_out,
                          void* ws, hipStream_t stream);
hipError_t launch_decode(const void* q, const void* k, const void* v, void* o, float* S, float* z, int BH, int D,
                         int M, int bf16, hipStream_t stream);
hipError_t launch_deltanet(const void* q, const void* k, const void* v, const void* beta, void* o, int BH, int N,
                           int D, int M, int bf16, const float* W0, float* W_out, void* ws, hipStream_t stream);
// Chunk-parallel delta rule (prep, scan and output kernels) and the workspace it needs.
size_t deltanet_chunk_ws_bytes(int BH, int N, int D, int M);
hipError_t launch_deltanet_chunked(const void* q, const void* k, const void* v, const void* beta, void* o, int BH,
                                   int N, int D, int M, int bf16, const float* W0, float* W_out, void* ws,
                                   hipStream_t stream);
size_t deltanet_ws_bytes(int BH, int N, int D, int M);
// Device address of the current GPU's copy of the library-owned scratch array
// (LINATTN_NOALLOC_SCRATCH_BYTES bytes), or NULL if it cannot be obtained.
void* noalloc_scratch();
hipError_t launch_deltanet_step(const void* q, const void* k, const void* v, const void* beta, void* o, float* W,
                                int BH, int D, int M, int bf16, hipStream_t stream);

}  // namespace la
