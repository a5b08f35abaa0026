// focus_selftest.hip -- test-only library: runs the quantizer's device
// arithmetic helpers (fp4_post_weight_amd/csrc/focus_numerics.h) on the GPU,
// either exhaustively over binary32 inputs against an independent device
// formulation of the same rule, or over host-given arrays so the GPU tests can
// compare them with the CPU oracle.  Loaded only by tests/test_gpu_helpers.py.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "focus_numerics.h"

using namespace focus;

namespace {

constexpr int kT = 256;
constexpr unsigned kGrid = 16384;

__device__ unsigned long long g_result;

__device__ __forceinline__ uint64_t gtid() { return (uint64_t)blockIdx.x * kT + threadIdx.x; }
__device__ __forceinline__ uint64_t gstride() { return (uint64_t)gridDim.x * kT; }

// E2M1 from its definition: clamp to [-6, 6], nearest magnitude, ties to the
// even code; sign bit = sign of the input.
__device__ unsigned e2m1_reference(float x) {
    const double mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
    const unsigned sign = __float_as_uint(x) >> 31;
    double a = fabs((double)x);
    if (a > 6.0) a = 6.0;
    unsigned best = 0;
    double bd = 1e300;
    for (unsigned k = 0; k < 8; ++k) {
        const double d = fabs(a - mag[k]);
        if (d < bd || (d == bd && (k & 1u) == 0u)) {
            bd = d;
            best = k;
        }
    }
    return (sign << 3) | best;
}

// BF16 round to nearest even by integer arithmetic on the bits (finite x).
__device__ uint32_t bf16_reference(float x) {
    uint32_t b = __float_as_uint(x);
    if ((b & 0x7F800000u) == 0x7F800000u) return b >> 16;  // infinities
    return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

// 0: corrected hardware reciprocal vs IEEE division, every s in [1, 2^126)
__global__ void k_recip(unsigned long long* bad) {
    const uint64_t lo = 0x3F800000u, hi = 0x7E800000u;  // [1, 2^126)
    unsigned long long n = 0;
    for (uint64_t i = gtid(); i < hi - lo; i += gstride()) {
        const float s = __uint_as_float((uint32_t)(lo + i));
        if (__float_as_uint(recip_rn_ge1(s)) != __float_as_uint(1.0f / s)) ++n;
    }
    if (n) atomicAdd(bad, n);
}

// 1: largest |r*d - 1| of recip_f64 over every positive finite binary32 d
// (returned as the bits of a non-negative double: integer order = value order)
__global__ void k_rcp64(unsigned long long* maxbits) {
    double m = 0.0;
    for (uint64_t i = gtid(); i < 0x7F7FFFFFull; i += gstride()) {
        const double d = (double)__uint_as_float((uint32_t)i + 1u);
        m = fmax(m, fabs(__builtin_fma(recip_f64(d), d, -1.0)));
    }
    atomicMax(maxbits, (unsigned long long)__double_as_longlong(m));
}

// 2: exp_f64 rounded to binary32 vs the platform binary64 exp rounded to
// binary32, every binary32 x in [-105, 89]
__global__ void k_exp(unsigned long long* bad) {
    const uint64_t npos = 0x42B20000ull + 1, nneg = 0x42D20000ull + 1;
    unsigned long long n = 0;
    for (uint64_t i = gtid(); i < npos + nneg; i += gstride()) {
        const uint32_t p = i < npos ? (uint32_t)i : (0x80000000u | (uint32_t)(i - npos));
        const double x = (double)__uint_as_float(p);
        if (__float_as_uint((float)exp_f64(x, kExp2Frac64)) != __float_as_uint((float)exp(x))) ++n;
    }
    if (n) atomicAdd(bad, n);
}

// 3: hardware E2M1 packing (both nibble slots) vs the definition, every
// non-NaN binary32
__global__ void k_e2m1(unsigned long long* bad) {
    unsigned long long n = 0;
    for (uint64_t i = gtid(); i < (1ull << 31); i += gstride()) {
        const float x = __uint_as_float((uint32_t)i);
        if (x != x) continue;
        const float y = -x;
        float v[8] = {x, y, y, x, x, y, y, x};
        const uint32_t c = pack8(v);
        const uint32_t cx = e2m1_reference(x), cy = e2m1_reference(y);
        const uint32_t want = cx | (cy << 4) | (cy << 8) | (cx << 12) | (cx << 16) | (cy << 20) |
                              (cy << 24) | (cx << 28);
        if (c != want) ++n;
    }
    if (n) atomicAdd(bad, n);
}

// 4: hardware BF16 pair conversion vs integer RNE, every non-NaN binary32
__global__ void k_bf16(unsigned long long* bad) {
    unsigned long long n = 0;
    for (uint64_t i = gtid(); i < (1ull << 31); i += gstride()) {
        const float x = __uint_as_float((uint32_t)i);
        if (x != x) continue;
        const float y = -x;
        const uint32_t got = bf16_pair(x, y);
        const uint32_t want = bf16_reference(x) | (bf16_reference(y) << 16);
        if (got != want) ++n;
    }
    if (n) atomicAdd(bad, n);
}

// array maps ------------------------------------------------------------------

__global__ void m_e2m1(const float* x, int64_t n, uint8_t* out) {  // n even
    for (uint64_t i = gtid(); i < (uint64_t)n / 2; i += gstride()) {
        float v[8] = {x[2 * i], x[2 * i + 1], 0, 0, 0, 0, 0, 0};
        const uint32_t c = pack8(v);
        out[2 * i] = c & 15u;
        out[2 * i + 1] = (c >> 4) & 15u;
    }
}
__global__ void m_bf16(const float* x, int64_t n, uint16_t* out) {  // n even
    for (uint64_t i = gtid(); i < (uint64_t)n / 2; i += gstride()) {
        const uint32_t h = bf16_pair(x[2 * i], x[2 * i + 1]);
        out[2 * i] = (uint16_t)(h & 0xFFFFu);
        out[2 * i + 1] = (uint16_t)(h >> 16);
    }
}
__global__ void m_sigmoid(const float* q, int64_t n, float* out) {
    for (uint64_t i = gtid(); i < (uint64_t)n; i += gstride()) out[i] = sigmoid_cr(q[i], kExp2Frac64);
}
__global__ void m_expf(const float* x, int64_t n, float* out) {
    for (uint64_t i = gtid(); i < (uint64_t)n; i += gstride())
        out[i] = (float)exp_f64((double)x[i], kExp2Frac64);
}
__global__ void m_e4m3(const float* t, int64_t n, uint8_t* out) {  // t in [2^-6, 448]
    for (uint64_t i = gtid(); i < (uint64_t)n; i += gstride()) out[i] = (uint8_t)e4m3_byte_normal(t[i]);
}
// element quotient as the quantizer forms it: x = RN32(RN64(w * recip_f64(d)))
__global__ void m_quot(const float* w, const float* d, int64_t n, float* out) {
    for (uint64_t i = gtid(); i < (uint64_t)n; i += gstride())
        out[i] = (float)((double)w[i] * recip_f64((double)d[i]));
}
// block quotient t as the quantizer forms it from num and den
__global__ void m_blockt(const float* num, const float* den, int64_t n, float* out) {
    for (uint64_t i = gtid(); i < (uint64_t)n; i += gstride())
        out[i] = (float)((double)num[i] * (1.0 / (double)den[i]));
}

}  // namespace

extern "C" {

// Exhaustive check `which` (0..4, see the kernels above); *result receives the
// mismatch count (or, for 1, the bits of the largest residual).  Synchronous.
int focus_selftest_exhaustive(int which, unsigned long long* result) {
    unsigned long long* d = nullptr;
    if (hipMalloc(&d, sizeof(*d)) != hipSuccess) return 1;
    hipMemset(d, 0, sizeof(*d));
    switch (which) {
        case 0: hipLaunchKernelGGL(k_recip, dim3(kGrid), dim3(kT), 0, 0, d); break;
        case 1: hipLaunchKernelGGL(k_rcp64, dim3(kGrid), dim3(kT), 0, 0, d); break;
        case 2: hipLaunchKernelGGL(k_exp, dim3(kGrid), dim3(kT), 0, 0, d); break;
        case 3: hipLaunchKernelGGL(k_e2m1, dim3(kGrid), dim3(kT), 0, 0, d); break;
        case 4: hipLaunchKernelGGL(k_bf16, dim3(kGrid), dim3(kT), 0, 0, d); break;
        default: hipFree(d); return 2;
    }
    hipError_t e = hipMemcpy(result, d, sizeof(*d), hipMemcpyDeviceToHost);
    hipFree(d);
    return e == hipSuccess ? 0 : 1;
}

// Map `which` over n device elements (synchronous).  0: E2M1 codes (uint8 out,
// n even), 1: BF16 (uint16 out, n even), 2: sigmoid, 3: expf, 4: E4M3 byte of
// t in [2^-6, 448], 5: element quotient (in2 = d), 6: block quotient
// (in = num, in2 = den).
int focus_selftest_map(int which, const void* in, const void* in2, void* out, int64_t n) {
    const dim3 g(kGrid), b(kT);
    const float* x = (const float*)in;
    switch (which) {
        case 0: hipLaunchKernelGGL(m_e2m1, g, b, 0, 0, x, n, (uint8_t*)out); break;
        case 1: hipLaunchKernelGGL(m_bf16, g, b, 0, 0, x, n, (uint16_t*)out); break;
        case 2: hipLaunchKernelGGL(m_sigmoid, g, b, 0, 0, x, n, (float*)out); break;
        case 3: hipLaunchKernelGGL(m_expf, g, b, 0, 0, x, n, (float*)out); break;
        case 4: hipLaunchKernelGGL(m_e4m3, g, b, 0, 0, x, n, (uint8_t*)out); break;
        case 5: hipLaunchKernelGGL(m_quot, g, b, 0, 0, x, (const float*)in2, n, (float*)out); break;
        case 6: hipLaunchKernelGGL(m_blockt, g, b, 0, 0, x, (const float*)in2, n, (float*)out); break;
        default: return 2;
    }
    return hipDeviceSynchronize() == hipSuccess ? 0 : 1;
}

}  // extern "C"
