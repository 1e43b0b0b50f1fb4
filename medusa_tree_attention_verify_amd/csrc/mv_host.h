// Host-side helpers of the C ABI: status codes, workspace carving, launch checks.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "medusa_verify.h"

namespace mv {

constexpr size_t kAlign = 256;

inline size_t align_up(size_t x, size_t a = kAlign) { return (x + a - 1) / a * a; }

// Sequential carving of one caller-provided workspace into aligned sub-buffers.  With
// base == nullptr it only measures.
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base(static_cast<char*>(b)) {}
  template <typename T>
  T* take(size_t count) {
    off = align_up(off);
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += count * sizeof(T);
    return p;
  }
  size_t bytes() const { return align_up(off); }
};

inline int check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return MV_OK;
  if (ws == nullptr || ws_bytes < need) return MV_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(ws) % kAlign) return MV_ERR_WORKSPACE;
  return MV_OK;
}

inline int launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? MV_OK : MV_ERR_HIP;
}

inline hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

inline int ceil_div(long long a, long long b) { return static_cast<int>((a + b - 1) / b); }

// Internal (lmhead.hip): rows_out[t][v] = exp(W[v] . x[row(t)] - lse_in[row(t)]) for T target
// rows, row(t) = t * xrow_mul + xrow[t * xrow_stride] (xrow null: t); bf16 x and W, d % 32 == 0.
int lm_head_prob_rows(int T, int d, int V, const uint16_t* x, const int* xrow, int xrow_stride,
                      int xrow_mul, const float* lse_in, const uint16_t* w, float* rows_out,
                      hipStream_t st);

}  // namespace mv

#define MV_TRY(expr)            \
  do {                          \
    int _st = (expr);           \
    if (_st != MV_OK) return _st; \
  } while (0)
