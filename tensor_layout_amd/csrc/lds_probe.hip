// lds_probe.hip -- measure the LDS bank geometry the planner's bank model uses.
//
// Run it under the LDS bank-conflict counter, e.g.
//   rocprofv3 --pmc SQ_LDS_BANK_CONFLICT SQ_INSTS_LDS -d <dir> -o p -- ./lds_probe
// Every test is one dispatch of one wave whose grid size (in workgroups) is
// the test number, so a counter row maps back to the line this program
// prints for that test.  A test repeats one LDS access 64 times.
//
// Two-lane tests (only lanes 0 and B access LDS, lane 0 at byte 0, lane B at
// byte X) tell, for each instruction:
//   kind=bank: B = 1, X over every multiple of the access width up to twice
//              the largest candidate bank period -> conflicts repeat with the
//              bank period (banks x 4 bytes);
//   kind=pass: X = one bank period, B over every lane -> lane B conflicts with
//              lane 0 exactly when both are served in the same pass.
// Whole-wave tests (kind=tile) run the tiled kernel's 16-byte read map: lane
// L reads row L%8 at a given pitch, column L/8.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#define PROBE_CHECK(x)                                                                       \
    do {                                                                                     \
        hipError_t e_ = (x);                                                                 \
        if (e_ != hipSuccess) {                                                              \
            std::fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
            std::exit(1);                                                                    \
        }                                                                                    \
    } while (0)

constexpr int kLdsBytes = 65536;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// addrs: byte address per lane, or 0xffffffff for a lane that does not access LDS.
template <int W, bool WRITE>
__global__ void __launch_bounds__(64) probe_kernel(const uint32_t* __restrict__ addrs, uint32_t* __restrict__ sink) {
    __shared__ __attribute__((aligned(16))) uint32_t lds[kLdsBytes / 4];
    const int lane = threadIdx.x;
    for (int i = lane; i < 1024; i += 64) lds[i] = i;
    __syncthreads();
    const uint32_t a = addrs[lane];
    uint32_t acc = 0;
    if (a != 0xffffffffu) {
        const uint32_t p = (uint32_t)(uintptr_t)lds + a;
        for (int it = 0; it < 64; ++it) {
            if constexpr (WRITE) {
                if constexpr (W == 16) {
                    u32x4 v = {acc, acc, acc, acc};
                    asm volatile("ds_write_b128 %0, %1\n s_waitcnt lgkmcnt(0)" ::"v"(p), "v"(v) : "memory");
                } else if constexpr (W == 8) {
                    uint64_t v = acc;
                    asm volatile("ds_write_b64 %0, %1\n s_waitcnt lgkmcnt(0)" ::"v"(p), "v"(v) : "memory");
                } else {
                    asm volatile("ds_write_b32 %0, %1\n s_waitcnt lgkmcnt(0)" ::"v"(p), "v"(acc) : "memory");
                }
            } else {
                if constexpr (W == 16) {
                    u32x4 v;
                    asm volatile("ds_read_b128 %0, %1\n s_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(p) : "memory");
                    acc += v.x ^ v.w;
                } else if constexpr (W == 8) {
                    uint64_t v;
                    asm volatile("ds_read_b64 %0, %1\n s_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(p) : "memory");
                    acc += (uint32_t)v;
                } else {
                    uint32_t v;
                    asm volatile("ds_read_b32 %0, %1\n s_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(p) : "memory");
                    acc += v;
                }
            }
        }
    }
    sink[blockIdx.x * 64 + lane] = acc;
}

struct Test {
    int w;
    bool write;
    const char* kind;
    int B;
    uint32_t X;
    int pitch;
    std::vector<uint32_t> addrs;
};

int main() {
    std::vector<Test> tests;
    const uint32_t kOff = 0xffffffffu;
    for (bool wr : {false, true}) {
        for (int w : {4, 8, 16}) {
            // bank period: lane 1 over multiples of w up to 512 bytes
            for (uint32_t X = w; X <= 512; X += w) {
                Test t{w, wr, "bank", 1, X, 0, std::vector<uint32_t>(64, kOff)};
                t.addrs[0] = 0;
                t.addrs[1] = X;
                tests.push_back(t);
            }
            // pass membership: lane B at 512 bytes (a multiple of every candidate period)
            for (int B = 1; B < 64; ++B) {
                Test t{w, wr, "pass", B, 512, 0, std::vector<uint32_t>(64, kOff)};
                t.addrs[0] = 0;
                t.addrs[B] = 512;
                tests.push_back(t);
            }
        }
    }
    for (int pitch : {1024, 1040, 1056, 1072, 1088, 1104, 1120, 1136, 1152, 1280, 272, 288, 304, 320}) {
        Test t{16, false, "tile", -1, 0, pitch, std::vector<uint32_t>(64)};
        for (int L = 0; L < 64; ++L) t.addrs[L] = (uint32_t)((L % 8) * pitch + (L / 8) * 16);
        tests.push_back(t);
    }
    uint32_t *d_addrs = nullptr, *d_sink = nullptr;
    PROBE_CHECK(hipMalloc(&d_addrs, 64 * sizeof(uint32_t)));
    PROBE_CHECK(hipMalloc(&d_sink, (tests.size() + 1) * 64 * sizeof(uint32_t)));
    for (size_t i = 0; i < tests.size(); ++i) {
        const Test& t = tests[i];
        for (uint32_t a : t.addrs) {
            if (a != kOff && (a % t.w || a + 16 > (uint32_t)kLdsBytes)) {
                std::fprintf(stderr, "test %zu: address out of range\n", i + 1);
                return 1;
            }
        }
        PROBE_CHECK(hipMemcpy(d_addrs, t.addrs.data(), 64 * sizeof(uint32_t), hipMemcpyHostToDevice));
        dim3 grid((unsigned)(i + 1)), block(64);
        if (t.write) {
            if (t.w == 16) probe_kernel<16, true><<<grid, block>>>(d_addrs, d_sink);
            else if (t.w == 8) probe_kernel<8, true><<<grid, block>>>(d_addrs, d_sink);
            else probe_kernel<4, true><<<grid, block>>>(d_addrs, d_sink);
        } else {
            if (t.w == 16) probe_kernel<16, false><<<grid, block>>>(d_addrs, d_sink);
            else if (t.w == 8) probe_kernel<8, false><<<grid, block>>>(d_addrs, d_sink);
            else probe_kernel<4, false><<<grid, block>>>(d_addrs, d_sink);
        }
        PROBE_CHECK(hipGetLastError());
        PROBE_CHECK(hipDeviceSynchronize());
        std::printf("test %zu op=%s bytes=%d kind=%s B=%d X=%u pitch=%d\n", i + 1, t.write ? "write" : "read", t.w,
                    t.kind, t.B, t.X, t.pitch);
    }
    std::fflush(stdout);
    return 0;
}
