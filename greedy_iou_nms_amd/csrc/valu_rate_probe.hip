// Issue cost of single VALU instructions on gfx950, for the roofline of the
// ALU-bound kernels (built by build.py next to the library; run by
// `bench.py --valu-rates`).  Each thread executes ITER x 16 instructions of
// one kind spread over 8 independent registers, with 4 or 8 waves per SIMD;
// the printed figure is cycles per wave64 instruction per SIMD at the
// nominal 2.4 GHz.  Every kernel writes one value per thread into a buffer
// sized for its grid, nothing else.
#include <hip/hip_runtime.h>
#include <cstdio>
#include <vector>
#define ITER 4096
#define BODY8(I) I(0) I(1) I(2) I(3) I(4) I(5) I(6) I(7)

#define F32_KERNEL(name, instr)                                                        \
__global__ __launch_bounds__(256) void name(float *out, float s) {                    \
    float r0 = threadIdx.x, r1 = r0 + 1, r2 = r0 + 2, r3 = r0 + 3, r4 = r0 + 4,        \
          r5 = r0 + 5, r6 = r0 + 6, r7 = r0 + 7;                                        \
    for (int i = 0; i < ITER; ++i) {                                                    \
        asm volatile(instr " %0, %8, %0\n" instr " %1, %8, %1\n" instr " %2, %8, %2\n"  \
                     instr " %3, %8, %3\n" instr " %4, %8, %4\n" instr " %5, %8, %5\n"  \
                     instr " %6, %8, %6\n" instr " %7, %8, %7\n"                        \
                     instr " %0, %8, %0\n" instr " %1, %8, %1\n" instr " %2, %8, %2\n"  \
                     instr " %3, %8, %3\n" instr " %4, %8, %4\n" instr " %5, %8, %5\n"  \
                     instr " %6, %8, %6\n" instr " %7, %8, %7\n"                        \
                     : "+v"(r0), "+v"(r1), "+v"(r2), "+v"(r3), "+v"(r4), "+v"(r5),      \
                       "+v"(r6), "+v"(r7) : "v"(s));                                    \
    }                                                                                   \
    out[blockIdx.x * 256 + threadIdx.x] = r0 + r1 + r2 + r3 + r4 + r5 + r6 + r7;        \
}
F32_KERNEL(k_add_f32, "v_add_f32")
F32_KERNEL(k_sub_f32, "v_sub_f32")
F32_KERNEL(k_mul_f32, "v_mul_f32")
F32_KERNEL(k_max_f32, "v_max_f32")
F32_KERNEL(k_fmac_f32, "v_fmac_f32")

#define F32_3OP(name, instr)                                                           \
__global__ __launch_bounds__(256) void name(float *out, float s) {                    \
    float r0 = threadIdx.x, r1 = r0 + 1, r2 = r0 + 2, r3 = r0 + 3, r4 = r0 + 4,        \
          r5 = r0 + 5, r6 = r0 + 6, r7 = r0 + 7;                                        \
    for (int i = 0; i < ITER; ++i) {                                                    \
        asm volatile(instr " %0, %8, %0, %8\n" instr " %1, %8, %1, %8\n" instr " %2, %8, %2, %8\n"  \
                     instr " %3, %8, %3, %8\n" instr " %4, %8, %4, %8\n" instr " %5, %8, %5, %8\n"  \
                     instr " %6, %8, %6, %8\n" instr " %7, %8, %7, %8\n"                        \
                     instr " %0, %8, %0, %8\n" instr " %1, %8, %1, %8\n" instr " %2, %8, %2, %8\n"  \
                     instr " %3, %8, %3, %8\n" instr " %4, %8, %4, %8\n" instr " %5, %8, %5, %8\n"  \
                     instr " %6, %8, %6, %8\n" instr " %7, %8, %7, %8\n"                        \
                     : "+v"(r0), "+v"(r1), "+v"(r2), "+v"(r3), "+v"(r4), "+v"(r5),      \
                       "+v"(r6), "+v"(r7) : "v"(s));                                    \
    }                                                                                   \
    out[blockIdx.x * 256 + threadIdx.x] = r0 + r1 + r2 + r3 + r4 + r5 + r6 + r7;        \
}
F32_3OP(k_med3_f32, "v_med3_f32")
F32_3OP(k_fma_f32, "v_fma_f32")
F32_3OP(k_max3_f32, "v_max3_f32")

// f64: 8 independent doubles
#define F64_KERNEL(name, instr)                                                        \
__global__ __launch_bounds__(256) void name(float *out, double s) {                   \
    double r0 = threadIdx.x, r1 = r0 + 1, r2 = r0 + 2, r3 = r0 + 3, r4 = r0 + 4,       \
           r5 = r0 + 5, r6 = r0 + 6, r7 = r0 + 7;                                       \
    for (int i = 0; i < ITER; ++i) {                                                    \
        asm volatile(instr " %0, %8, %0\n" instr " %1, %8, %1\n" instr " %2, %8, %2\n"  \
                     instr " %3, %8, %3\n" instr " %4, %8, %4\n" instr " %5, %8, %5\n"  \
                     instr " %6, %8, %6\n" instr " %7, %8, %7\n"                        \
                     instr " %0, %8, %0\n" instr " %1, %8, %1\n" instr " %2, %8, %2\n"  \
                     instr " %3, %8, %3\n" instr " %4, %8, %4\n" instr " %5, %8, %5\n"  \
                     instr " %6, %8, %6\n" instr " %7, %8, %7\n"                        \
                     : "+v"(r0), "+v"(r1), "+v"(r2), "+v"(r3), "+v"(r4), "+v"(r5),      \
                       "+v"(r6), "+v"(r7) : "v"(s));                                    \
    }                                                                                   \
    out[blockIdx.x * 256 + threadIdx.x] = (float)(r0 + r1 + r2 + r3 + r4 + r5 + r6 + r7); \
}
F64_KERNEL(k_mul_f64, "v_mul_f64")
F64_KERNEL(k_add_f64, "v_add_f64")

// cvt f64 <- f32 (8 independent outputs from 8 inputs)
__global__ __launch_bounds__(256) void k_cvt_f64(float *out, float s) {
    float a0 = threadIdx.x, a1 = a0 + 1, a2 = a0 + 2, a3 = a0 + 3;
    double d0 = 0, d1 = 0, d2 = 0, d3 = 0;
    for (int i = 0; i < ITER; ++i) {
        asm volatile("v_cvt_f64_f32 %0, %4\nv_cvt_f64_f32 %1, %5\nv_cvt_f64_f32 %2, %6\nv_cvt_f64_f32 %3, %7\n"
                     "v_cvt_f64_f32 %0, %5\nv_cvt_f64_f32 %1, %6\nv_cvt_f64_f32 %2, %7\nv_cvt_f64_f32 %3, %4\n"
                     "v_cvt_f64_f32 %0, %6\nv_cvt_f64_f32 %1, %7\nv_cvt_f64_f32 %2, %4\nv_cvt_f64_f32 %3, %5\n"
                     "v_cvt_f64_f32 %0, %7\nv_cvt_f64_f32 %1, %4\nv_cvt_f64_f32 %2, %5\nv_cvt_f64_f32 %3, %6\n"
                     : "+v"(d0), "+v"(d1), "+v"(d2), "+v"(d3) : "v"(a0), "v"(a1), "v"(a2), "v"(a3));
    }
    out[blockIdx.x * 256 + threadIdx.x] = (float)(d0 + d1 + d2 + d3) + s;
}

// compare f64 -> vcc (16 compares), result folded via s_or into an sgpr pair
__global__ __launch_bounds__(256) void k_cmp_f64(float *out, double s) {
    double r0 = threadIdx.x, r1 = r0 + 1;
    unsigned long long acc = 0;
    for (int i = 0; i < ITER; ++i) {
        unsigned long long m;
        asm volatile("v_cmp_gt_f64 vcc, %1, %2\nv_cmp_gt_f64 vcc, %2, %1\nv_cmp_gt_f64 vcc, %1, %2\nv_cmp_gt_f64 vcc, %2, %1\n"
                     "v_cmp_gt_f64 vcc, %1, %2\nv_cmp_gt_f64 vcc, %2, %1\nv_cmp_gt_f64 vcc, %1, %2\nv_cmp_gt_f64 vcc, %2, %1\n"
                     "v_cmp_gt_f64 vcc, %1, %2\nv_cmp_gt_f64 vcc, %2, %1\nv_cmp_gt_f64 vcc, %1, %2\nv_cmp_gt_f64 vcc, %2, %1\n"
                     "v_cmp_gt_f64 vcc, %1, %2\nv_cmp_gt_f64 vcc, %2, %1\nv_cmp_gt_f64 vcc, %1, %2\nv_cmp_gt_f64 vcc, %2, %1\n"
                     "s_mov_b64 %0, vcc\n"
                     : "=s"(m) : "v"(r0), "v"(r1) : "vcc");
        acc ^= m;
    }
    out[blockIdx.x * 256 + threadIdx.x] = (float)(acc & 1) + (float)s;
}

__device__ __forceinline__ unsigned wl(unsigned old, unsigned val, int lane) {
    asm volatile("v_writelane_b32 %0, %1, m0" : "+v"(old) : "s"(val), "{m0}"(lane));
    return old;
}
__global__ __launch_bounds__(256) void k_writelane(float *out, unsigned sv, unsigned sv2) {
    unsigned r[8];
    for (int q = 0; q < 8; ++q) r[q] = threadIdx.x + q;
    for (int i = 0; i < ITER; ++i) {
        const int ln = i & 63;
#pragma unroll
        for (int q = 0; q < 16; ++q) r[q & 7] = wl(r[q & 7], (q & 1) ? sv : sv2, ln);
    }
    unsigned t = 0;
    for (int q = 0; q < 8; ++q) t += r[q];
    out[blockIdx.x * 256 + threadIdx.x] = (float)t;
}

// integer / bit ops: 16 per iteration over 8 registers
#define U32_KERNEL(name, body)                                                          \
__global__ __launch_bounds__(256) void name(float *out, float s) {                      \
    unsigned r0 = threadIdx.x, r1 = r0 + 1, r2 = r0 + 2, r3 = r0 + 3, r4 = r0 + 4,      \
             r5 = r0 + 5, r6 = r0 + 6, r7 = r0 + 7;                                      \
    unsigned sv = (unsigned)(threadIdx.x * 3 + 1);                                      \
    for (int i = 0; i < ITER; ++i) {                                                    \
        asm volatile(body body : "+v"(r0), "+v"(r1), "+v"(r2), "+v"(r3), "+v"(r4),      \
                     "+v"(r5), "+v"(r6), "+v"(r7) : "v"(sv) : "vcc");                    \
    }                                                                                   \
    out[blockIdx.x * 256 + threadIdx.x] = (float)(r0 + r1 + r2 + r3 + r4 + r5 + r6 + r7) + s; \
}
#define ADDC8 "v_addc_co_u32 %0, vcc, %0, %0, vcc\nv_addc_co_u32 %1, vcc, %1, %1, vcc\nv_addc_co_u32 %2, vcc, %2, %2, vcc\nv_addc_co_u32 %3, vcc, %3, %3, vcc\nv_addc_co_u32 %4, vcc, %4, %4, vcc\nv_addc_co_u32 %5, vcc, %5, %5, vcc\nv_addc_co_u32 %6, vcc, %6, %6, vcc\nv_addc_co_u32 %7, vcc, %7, %7, vcc\n"
#define OR8 "v_or_b32 %0, %8, %0\nv_or_b32 %1, %8, %1\nv_or_b32 %2, %8, %2\nv_or_b32 %3, %8, %3\nv_or_b32 %4, %8, %4\nv_or_b32 %5, %8, %5\nv_or_b32 %6, %8, %6\nv_or_b32 %7, %8, %7\n"
U32_KERNEL(k_addc, ADDC8)
U32_KERNEL(k_or, OR8)
// two-operand (VOP2) and three-operand (VOP3) forms over the 8 registers
#define OP2_8(I) I " %0, %8, %0\n" I " %1, %8, %1\n" I " %2, %8, %2\n" I " %3, %8, %3\n" \
                 I " %4, %8, %4\n" I " %5, %8, %5\n" I " %6, %8, %6\n" I " %7, %8, %7\n"
#define OP3_8(I) I " %0, %8, %0, %8\n" I " %1, %8, %1, %8\n" I " %2, %8, %2, %8\n"         \
                 I " %3, %8, %3, %8\n" I " %4, %8, %4, %8\n" I " %5, %8, %5, %8\n"         \
                 I " %6, %8, %6, %8\n" I " %7, %8, %7, %8\n"
#define CMP_8(I) I " vcc, %8, %0\n" I " vcc, %8, %1\n" I " vcc, %8, %2\n" I " vcc, %8, %3\n" \
                 I " vcc, %8, %4\n" I " vcc, %8, %5\n" I " vcc, %8, %6\n" I " vcc, %8, %7\n"
#define CND_8 "v_cndmask_b32 %0, %0, %8, vcc\nv_cndmask_b32 %1, %1, %8, vcc\n"               \
              "v_cndmask_b32 %2, %2, %8, vcc\nv_cndmask_b32 %3, %3, %8, vcc\n"               \
              "v_cndmask_b32 %4, %4, %8, vcc\nv_cndmask_b32 %5, %5, %8, vcc\n"               \
              "v_cndmask_b32 %6, %6, %8, vcc\nv_cndmask_b32 %7, %7, %8, vcc\n"
U32_KERNEL(k_max_i32, OP2_8("v_max_i32"))
U32_KERNEL(k_min_u32, OP2_8("v_min_u32"))
U32_KERNEL(k_add_u32, OP2_8("v_add_u32"))
U32_KERNEL(k_sub_u32, OP2_8("v_sub_u32"))
U32_KERNEL(k_and_b32, OP2_8("v_and_b32"))
U32_KERNEL(k_lshl_b32, OP2_8("v_lshlrev_b32"))
U32_KERNEL(k_med3_i32, OP3_8("v_med3_i32"))
U32_KERNEL(k_max3_i32, OP3_8("v_max3_i32"))
U32_KERNEL(k_sub_f32_e64, OP2_8("v_sub_f32_e64"))
U32_KERNEL(k_cmp_gt_i32, CMP_8("v_cmp_gt_i32"))
U32_KERNEL(k_cmp_gt_f32, CMP_8("v_cmp_gt_f32"))
U32_KERNEL(k_cndmask, CND_8)

// rcp f32 (transcendental)
__global__ __launch_bounds__(256) void k_rcp_f32(float *out, float s) {
    float r0 = threadIdx.x + 1, r1 = r0 + 1, r2 = r0 + 2, r3 = r0 + 3, r4 = r0 + 4, r5 = r0 + 5, r6 = r0 + 6, r7 = r0 + 7;
    for (int i = 0; i < ITER; ++i) {
        asm volatile("v_rcp_f32 %0, %0\nv_rcp_f32 %1, %1\nv_rcp_f32 %2, %2\nv_rcp_f32 %3, %3\n"
                     "v_rcp_f32 %4, %4\nv_rcp_f32 %5, %5\nv_rcp_f32 %6, %6\nv_rcp_f32 %7, %7\n"
                     "v_rcp_f32 %0, %0\nv_rcp_f32 %1, %1\nv_rcp_f32 %2, %2\nv_rcp_f32 %3, %3\n"
                     "v_rcp_f32 %4, %4\nv_rcp_f32 %5, %5\nv_rcp_f32 %6, %6\nv_rcp_f32 %7, %7\n"
                     : "+v"(r0), "+v"(r1), "+v"(r2), "+v"(r3), "+v"(r4), "+v"(r5), "+v"(r6), "+v"(r7));
    }
    out[blockIdx.x * 256 + threadIdx.x] = r0 + r1 + r2 + r3 + r4 + r5 + r6 + r7 + s;
}

typedef void (*KF)(float *, float);
typedef void (*KD)(float *, double);
typedef void (*KW)(float *, unsigned, unsigned);

int main() {
    int cus = 0;
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, 0);
    int clk = 0;
    (void)hipDeviceGetAttribute(&clk, hipDeviceAttributeClockRate, 0);
    printf("CUs %d clock attr %d kHz\n", cus, clk);
    const int maxblocks = cus * 8;
    float *out;
    if (hipMalloc(&out, (size_t)maxblocks * 256 * 4) != hipSuccess) return 1;
    hipEvent_t e0, e1;
    (void)hipEventCreate(&e0);
    (void)hipEventCreate(&e1);
    struct { const char *name; KF f; KD d; KW w; } ks[] = {
        {"v_addc_co_u32", k_addc, nullptr}, {"v_or_b32", k_or, nullptr},
        {"v_writelane", nullptr, nullptr, k_writelane}, {"v_fmac_f32", k_fmac_f32, nullptr},
        {"v_add_f32", k_add_f32, nullptr}, {"v_sub_f32", k_sub_f32, nullptr},
        {"v_mul_f32", k_mul_f32, nullptr}, {"v_max_f32", k_max_f32, nullptr},
        {"v_med3_f32", k_med3_f32, nullptr}, {"v_fma_f32", k_fma_f32, nullptr},
        {"v_max3_f32", k_max3_f32, nullptr}, {"v_cvt_f64_f32", k_cvt_f64, nullptr},
{"v_rcp_f32", k_rcp_f32, nullptr},
        {"v_mul_f64", nullptr, k_mul_f64}, {"v_add_f64", nullptr, k_add_f64},
        {"v_cmp_gt_f64", nullptr, k_cmp_f64},
        {"v_max_i32", k_max_i32, nullptr}, {"v_min_u32", k_min_u32, nullptr},
        {"v_add_u32", k_add_u32, nullptr}, {"v_sub_u32", k_sub_u32, nullptr},
        {"v_and_b32", k_and_b32, nullptr}, {"v_lshlrev_b32", k_lshl_b32, nullptr},
        {"v_med3_i32", k_med3_i32, nullptr}, {"v_max3_i32", k_max3_i32, nullptr},
        {"v_sub_f32_e64", k_sub_f32_e64, nullptr}, {"v_cmp_gt_i32", k_cmp_gt_i32, nullptr},
        {"v_cmp_gt_f32", k_cmp_gt_f32, nullptr}, {"v_cndmask_b32", k_cndmask, nullptr},
    };
    for (int bpc : {4, 8}) {  // workgroups of 4 waves per CU: 4 -> 4 waves/SIMD, 8 -> 8
        const int blocks = cus * bpc;
        for (auto &k : ks) {
            for (int rep = 0; rep < 2; ++rep) {
                (void)hipEventRecord(e0, 0);
                if (k.f) hipLaunchKernelGGL(k.f, dim3(blocks), dim3(256), 0, 0, out, 1.0001f);
                else if (k.d) hipLaunchKernelGGL(k.d, dim3(blocks), dim3(256), 0, 0, out, 1.0001);
                else hipLaunchKernelGGL(k.w, dim3(blocks), dim3(256), 0, 0, out, 3u, 5u);
                (void)hipEventRecord(e1, 0);
                (void)hipEventSynchronize(e1);
                if (hipGetLastError() != hipSuccess) { printf("launch error\n"); return 1; }
                float ms = 0;
                (void)hipEventElapsedTime(&ms, e0, e1);
                if (rep == 1) {
                    const double wave_instrs = (double)blocks * 4 * ITER * 16;
                    const double per_simd = wave_instrs / (cus * 4.0);
                    const double cycles = ms * 1e-3 * 2.4e9;
                    printf("waves/SIMD %d  %-14s %8.3f ms  cycles per wave-instr per SIMD %.2f\n",
                           bpc, k.name, ms, cycles / per_simd);
                }
            }
        }
    }
    (void)hipFree(out);
    return 0;
}
