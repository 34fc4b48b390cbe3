// abi_client.cpp -- a plain C++ client of the permute library's C ABI, with
// no Python and no torch: device memory from hipMalloc, its own stream.
// Test infrastructure (driven by tests/test_gpu_c_abi.py).
//
// usage: abi_client IN OUT W RANK EXT... SS... DS... OFF_S OFF_D BATCH OUT_BYTES [MODE]
//   IN holds the source bytes; OUT receives OUT_BYTES of the destination,
//   which starts filled with 0xA5.  Prints the plan, then "ok" or an error.
//   MODE: absent for tpl_plan + tpl_permute; "swz:B,BASE,SHIFT:B,BASE,SHIFT"
//   (source, destination swizzle) for tpl_plan_swizzled +
//   tpl_permute_swizzled; "staged:K" for tpl_permute_staged with xor_k K.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "tpl.h"

#define HIP_OK(x)                                                                        \
    do {                                                                                 \
        hipError_t e_ = (x);                                                             \
        if (e_ != hipSuccess) {                                                          \
            std::fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
            return 3;                                                                    \
        }                                                                                \
    } while (0)

int main(int argc, char** argv) {
    if (argc < 5) return 2;
    const char* in_path = argv[1];
    const char* out_path = argv[2];
    const int w = std::atoi(argv[3]);
    const int rank = std::atoi(argv[4]);
    if (rank < 1 || rank > 8 || (argc != 5 + 3 * rank + 4 && argc != 5 + 3 * rank + 5)) {
        std::fprintf(stderr, "bad arguments\n");
        return 2;
    }
    std::vector<int64_t> ext(rank), ss(rank), ds(rank);
    for (int i = 0; i < rank; ++i) {
        ext[i] = std::atoll(argv[5 + i]);
        ss[i] = std::atoll(argv[5 + rank + i]);
        ds[i] = std::atoll(argv[5 + 2 * rank + i]);
    }
    const int64_t offs[2] = {std::atoll(argv[5 + 3 * rank]), std::atoll(argv[6 + 3 * rank])};
    const int64_t batch = std::atoll(argv[7 + 3 * rank]);
    const int64_t out_bytes = std::atoll(argv[8 + 3 * rank]);
    const char* mode = argc == 5 + 3 * rank + 5 ? argv[9 + 3 * rank] : "";
    tpl_swizzle zs{0, 0, 0}, zd{0, 0, 0};
    bool swizzled = false, staged = false;
    int xor_k = -1;
    if (std::sscanf(mode, "swz:%d,%d,%d:%d,%d,%d", &zs.bits, &zs.base, &zs.shift, &zd.bits, &zd.base, &zd.shift) == 6) {
        swizzled = true;
    } else if (std::sscanf(mode, "staged:%d", &xor_k) == 1) {
        staged = true;
    } else if (mode[0]) {
        std::fprintf(stderr, "bad mode %s\n", mode);
        return 2;
    }

    std::FILE* f = std::fopen(in_path, "rb");
    if (!f) return 2;
    std::vector<uint8_t> host_in;
    uint8_t buf[1 << 16];
    size_t got;
    while ((got = std::fread(buf, 1, sizeof buf, f)) > 0) host_in.insert(host_in.end(), buf, buf + got);
    std::fclose(f);

    tpl_plan_info info;
    int st = swizzled ? tpl_plan_swizzled(w, rank, ext.data(), ss.data(), ds.data(), offs, batch, &zs, &zd,
                                          TPL_GEOM_GFX950, &info)
             : staged ? tpl_plan(w, rank, ext.data(), ss.data(), ds.data(), nullptr, 1, TPL_GEOM_GFX950_HALFWAVE, &info)
                      : tpl_plan(w, rank, ext.data(), ss.data(), ds.data(), offs, batch, TPL_GEOM_GFX950, &info);
    std::printf("plan status=%d kernel=%d tile=%dx%d k=%d grid=%lld block=%lld\n", st, info.kernel, info.tile[0],
                info.tile[1], info.k, (long long)info.grid, (long long)info.block);
    if (st != TPL_OK && !(staged && st == TPL_E_NO_K && xor_k >= 0)) {
        std::printf("declined: %s (%s)\n", tpl_status_string(st), tpl_last_error());
        return 4;
    }

    void *d_in = nullptr, *d_out = nullptr;
    HIP_OK(hipMalloc(&d_in, host_in.size() ? host_in.size() : 1));
    HIP_OK(hipMalloc(&d_out, out_bytes ? out_bytes : 1));
    HIP_OK(hipMemcpy(d_in, host_in.data(), host_in.size(), hipMemcpyHostToDevice));
    HIP_OK(hipMemset(d_out, 0xA5, out_bytes));
    hipStream_t stream;
    HIP_OK(hipStreamCreate(&stream));
    if (swizzled)
        st = tpl_permute_swizzled(d_in, d_out, w, rank, ext.data(), ss.data(), ds.data(), offs, batch, &zs, &zd, stream);
    else if (staged)
        st = tpl_permute_staged(d_in, d_out, w, rank, ext.data(), ss.data(), ds.data(), offs, batch, nullptr, nullptr,
                                xor_k, stream);
    else
        st = tpl_permute(d_in, d_out, w, rank, ext.data(), ss.data(), ds.data(), offs, batch, stream);
    if (st != TPL_OK) {
        std::printf("permute failed: %s (%s)\n", tpl_status_string(st), tpl_last_error());
        return 5;
    }
    HIP_OK(hipStreamSynchronize(stream));
    std::vector<uint8_t> host_out(out_bytes);
    HIP_OK(hipMemcpy(host_out.data(), d_out, out_bytes, hipMemcpyDeviceToHost));
    HIP_OK(hipStreamDestroy(stream));
    HIP_OK(hipFree(d_in));
    HIP_OK(hipFree(d_out));
    f = std::fopen(out_path, "wb");
    if (!f) return 2;
    std::fwrite(host_out.data(), 1, host_out.size(), f);
    std::fclose(f);
    std::printf("ok\n");
    return 0;
}
