// Drives the library's C ABI from a program whose host code (the library's
// included) is built with AddressSanitizer, so that the argument checks, the
// per-stream workspaces (growth, epochs, release), the static scratch and
// the dispatch tables run under it.
//
//   abi_asan host    argument checks and host-only calls (no GPU needed)
//   abi_asan device  the same, then scans, compactions, radix passes and CSR
//                    offsets on the GPU at sizes that grow each workspace
//                    several times, on two streams, with releases between
//
// Exit status 0 when every returned status and every checked output is as
// expected; AddressSanitizer ends the program with its own status on an error.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "dwpt_scan.h"

static int g_fail = 0;

#define EXPECT(cond)                                                          \
    do {                                                                      \
        if (!(cond)) {                                                        \
            std::fprintf(stderr, "%s:%d: expected %s\n", __FILE__, __LINE__, #cond); \
            ++g_fail;                                                         \
        }                                                                     \
    } while (0)

static void host_checks()
{
    alignas(16) static uint32_t buf[64];
    void* odd = reinterpret_cast<char*>(buf) + 2;
    // argument checks that return before any device work
    EXPECT(scan_inclusive(SCAN_OP_ADD, SCAN_I32, nullptr, buf, 10, nullptr) == SCAN_ERR_INVALID);
    EXPECT(scan_inclusive(SCAN_OP_ADD, SCAN_I32, buf, nullptr, 10, nullptr) == SCAN_ERR_INVALID);
    EXPECT(scan_inclusive(SCAN_OP_ADD, SCAN_I32, odd, buf, 10, nullptr) == SCAN_ERR_INVALID);
    EXPECT(scan_exclusive(SCAN_OP_ADD, SCAN_I32, buf, buf + 1, 16, nullptr) == SCAN_ERR_INVALID);  // partial overlap
    EXPECT(scan_inclusive((scan_op_t)99, SCAN_I32, buf, buf, 1, nullptr) == SCAN_ERR_UNSUPPORTED);
    EXPECT(scan_inclusive(SCAN_OP_ADD, (scan_dtype_t)99, buf, buf, 1, nullptr) == SCAN_ERR_UNSUPPORTED);
    EXPECT(scan_inclusive(SCAN_OP_AFFINE, SCAN_F32, buf, buf, 1, nullptr) == SCAN_ERR_UNSUPPORTED);
    EXPECT(segmented_scan(SCAN_OP_ADD, SCAN_I32, buf, nullptr, buf, 10, 0, nullptr) == SCAN_ERR_INVALID);
    EXPECT(compact(SCAN_F32, buf, buf + 32, buf, 4, nullptr) == SCAN_ERR_INVALID);       // count inside the input
    EXPECT(compact(SCAN_F32, buf, buf + 32, buf + 33, 8, nullptr) == SCAN_ERR_INVALID);  // count inside the output
    EXPECT(compact(SCAN_F32, buf, buf + 32, nullptr, 8, nullptr) == SCAN_ERR_INVALID);
    EXPECT(radix_split(buf, nullptr, 16, 32, buf + 32, nullptr, nullptr) == SCAN_ERR_INVALID);  // shift past the key
    EXPECT(radix_split(buf, buf + 16, 16, 0, buf + 32, nullptr, nullptr) == SCAN_ERR_INVALID);  // values without output
    EXPECT(radix_split(buf, nullptr, 16, 0, buf + 8, nullptr, nullptr) == SCAN_ERR_INVALID);    // output overlaps keys
    EXPECT(csr_row_offsets(buf, 4, 3, nullptr, nullptr) == SCAN_ERR_INVALID);
    EXPECT(scan_noalloc(SCAN_OP_MAT3, SCAN_U32X9, buf, buf, (size_t)1 << 40, 0, nullptr) == SCAN_ERR_INVALID);
    // strings and knobs
    for (int s = -1; s <= 7; ++s) EXPECT(std::strlen(scan_status_string((scan_status_t)s)) > 0);
    const size_t old = scan_set_small_n_max(123);
    EXPECT(scan_set_small_n_max(old) == 123);
    const int mode = scan_set_multi_tile_mode(2);
    EXPECT(scan_set_multi_tile_mode(mode) == 2);
    const uint32_t spin = scan_set_spin_limit(77);
    EXPECT(scan_set_spin_limit(spin) == 77);
}

#define HIPCHECK(x)                                                                       \
    do {                                                                                  \
        if ((x) != hipSuccess) {                                                          \
            std::fprintf(stderr, "%s:%d: %s failed\n", __FILE__, __LINE__, #x);           \
            std::exit(3);                                                                 \
        }                                                                                 \
    } while (0)

static void device_checks()
{
    int ndev = 0;
    HIPCHECK(hipGetDeviceCount(&ndev));
    EXPECT(ndev >= 1);
    hipStream_t s[2];
    HIPCHECK(hipStreamCreate(&s[0]));
    HIPCHECK(hipStreamCreate(&s[1]));
    const size_t nmax = (size_t)1 << 24;
    int32_t *x, *y;
    uint32_t *cnt, *keys, *kout, *rowp;
    uint8_t* heads;
    HIPCHECK(hipMalloc(&x, nmax * 4));
    HIPCHECK(hipMalloc(&y, nmax * 4));
    HIPCHECK(hipMalloc(&cnt, 4));
    HIPCHECK(hipMalloc(&keys, nmax * 4));
    HIPCHECK(hipMalloc(&kout, nmax * 4));
    HIPCHECK(hipMalloc(&heads, nmax));
    HIPCHECK(hipMalloc(&rowp, ((size_t)1 << 16) * 4 + 4));
    std::vector<int32_t> hx(nmax);
    for (size_t i = 0; i < nmax; ++i) hx[i] = (int32_t)(i % 7) - 3;
    std::vector<uint32_t> hk(nmax);
    for (size_t i = 0; i < nmax; ++i) hk[i] = (uint32_t)(i * 2654435761u) % (1u << 16);
    HIPCHECK(hipMemcpy(x, hx.data(), nmax * 4, hipMemcpyHostToDevice));
    HIPCHECK(hipMemcpy(keys, hk.data(), nmax * 4, hipMemcpyHostToDevice));
    HIPCHECK(hipMemset(heads, 0, nmax));
    for (int round = 0; round < 2; ++round) {
        // sizes that grow every workspace several times; both streams; every kernel path
        for (size_t n : {(size_t)1, (size_t)1000, (size_t)20000, (size_t)1 << 20, nmax}) {
            for (int mode : {0, 1, 2, 3}) {
                const int old = scan_set_multi_tile_mode(mode);
                hipStream_t st = s[(n + mode) % 2];
                EXPECT(scan_inclusive(SCAN_OP_ADD, SCAN_I32, x, y, n, st) == SCAN_OK);
                EXPECT(scan_exclusive(SCAN_OP_MAX, SCAN_I32, x, y, n, st) == SCAN_OK);
                EXPECT(segmented_scan(SCAN_OP_ADD, SCAN_I32, x, heads, y, n, 0, st) == SCAN_OK);
                EXPECT(compact(SCAN_I32, x, y, cnt, n, st) == SCAN_OK);
                scan_set_multi_tile_mode(old);
            }
            EXPECT(scan_noalloc(SCAN_OP_ADD, SCAN_I32, x, y, n, 1, s[0]) == SCAN_OK);
            EXPECT(radix_split(keys, nullptr, n, 8, kout, nullptr, s[1]) == SCAN_OK);
            if (n >= 2)
                EXPECT(radix_split(keys, keys + n / 2, n / 2, 0, kout, kout + n / 2, s[0]) == SCAN_OK);
            EXPECT(csr_row_offsets(kout, n, 1u << 16, rowp, s[1]) == SCAN_OK);
            HIPCHECK(hipDeviceSynchronize());
            EXPECT(scan_get_device_error(s[0]) == SCAN_OK);
            EXPECT(scan_get_device_error(s[1]) == SCAN_OK);
            // the last inclusive sum over the full size, against the host
            EXPECT(scan_inclusive(SCAN_OP_ADD, SCAN_I32, x, y, n, s[0]) == SCAN_OK);
            HIPCHECK(hipStreamSynchronize(s[0]));
            int32_t last = 0;
            HIPCHECK(hipMemcpy(&last, y + (n - 1), 4, hipMemcpyDeviceToHost));
            int64_t want = 0;
            for (size_t i = 0; i < n; ++i) want += hx[i];
            EXPECT(last == (int32_t)want);
        }
        EXPECT(scan_release_workspace() == SCAN_OK);
    }
    HIPCHECK(hipFree(x));
    HIPCHECK(hipFree(y));
    HIPCHECK(hipFree(cnt));
    HIPCHECK(hipFree(keys));
    HIPCHECK(hipFree(kout));
    HIPCHECK(hipFree(heads));
    HIPCHECK(hipFree(rowp));
    HIPCHECK(hipStreamDestroy(s[0]));
    HIPCHECK(hipStreamDestroy(s[1]));
}

int main(int argc, char** argv)
{
    const bool device = argc > 1 && std::strcmp(argv[1], "device") == 0;
    host_checks();
    if (device) device_checks();
    std::printf("abi_asan %s: %d failed checks\n", device ? "device" : "host", g_fail);
    return g_fail ? 1 : 0;
}
