# Fiber context switch for the CPU emulation of the HIP kernels (x86-64
# System V).  emu_switch(void** save_sp, void* load_sp) saves the callee-saved
# registers on the current stack, stores the stack pointer in *save_sp and
# resumes the context whose stack pointer is load_sp.  A fresh fiber's stack
# holds six zero register slots and the address of emu_fiber_tramp.
    .text
    .globl emu_switch
    .type emu_switch, @function
emu_switch:
    pushq %rbp
    pushq %rbx
    pushq %r12
    pushq %r13
    pushq %r14
    pushq %r15
    movq %rsp, (%rdi)
    movq %rsi, %rsp
    popq %r15
    popq %r14
    popq %r13
    popq %r12
    popq %rbx
    popq %rbp
    ret
    .size emu_switch, .-emu_switch

    .globl emu_fiber_tramp
    .type emu_fiber_tramp, @function
emu_fiber_tramp:
    andq $-16, %rsp
    call emu_fiber_main
    ud2
    .size emu_fiber_tramp, .-emu_fiber_tramp

    .section .note.GNU-stack,"",@progbits
