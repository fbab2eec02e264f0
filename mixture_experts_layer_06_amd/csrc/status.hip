// Status codes, thread-local error text and cached device properties.
#include <mutex>

#include "common.hpp"

namespace moe {

static thread_local std::string g_last_error;

void set_error(const std::string &msg) { g_last_error = msg; }
void clear_error() { g_last_error.clear(); }

int check_launch(const char *what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        set_error(std::string(what) + ": " + hipGetErrorString(e));
        return MOE_ERR_HIP;
    }
    return MOE_OK;
}

int num_cus() {
    static std::mutex mu;
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    std::lock_guard<std::mutex> lock(mu);
    if (cache[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cache[dev] = n;
    }
    return cache[dev];
}

}  // namespace moe

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char *moe_status_string(int status) {
    switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported size or option";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_HIP: return "HIP launch failure";
    default: return "unknown status";
    }
}

const char *moe_last_error(void) { return moe::g_last_error.c_str(); }

}  // extern "C"
